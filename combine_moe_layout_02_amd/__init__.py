"""MI355X-native MoE normal-mode layout / dispatch / combine.

Thin Python binding of ``libmoe.so`` (the HIP kernels behind the C ABI of
``include/moe.h``). Functions carry the C names; they only marshal torch tensors
(device pointers, sizes, the current HIP stream) into the C calls, allocate
outputs the caller did not pass, and turn negative status codes into
exceptions. Every step of the computation runs in the library's kernels; there
is no other code path. Importing this package fails if the library is not built
(``python combine_moe_layout_02_amd/build.py``).
"""

import ctypes
import os
from typing import NamedTuple

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
MOE_ERR_ARG = -1
MOE_ERR_ALIGN = -2
MOE_ERR_WINDOW = -3
MOE_ERR_UNSUPPORTED = -4
MOE_ERR_HIP = -5
MOE_ERR_SCRATCH = -6
MOE_NOALLOC_SCRATCH_BYTES = 1 << 20

MOE_QUANT_NONE = 0
MOE_QUANT_FP8_E4M3_DYN = 1
MOE_QUANT_INT8_DYN = 2

MOE_LAYOUT_AUTO = 0
MOE_LAYOUT_MULTI = 1
MOE_LAYOUT_SINGLE = 2

EXPORTED = (
    "moe_slot_bytes", "moe_window_bytes", "moe_slot_offsets", "moe_layout", "moe_layout_ex", "moe_dispatch",
    "moe_dispatch_workspace_bytes", "moe_dispatch_ws", "moe_dispatch_noalloc",
    "moe_layout_dispatch", "moe_layout_dispatch_ex", "moe_layout_dispatch_workspace_bytes",
    "moe_layout_ws", "moe_dispatch_planned", "moe_layout_dispatch_ws", "moe_combine", "moe_combine_scatter", "moe_combine_staged",
    "moe_unpack", "moe_unpack_padded", "moe_dedup_window_bytes", "moe_rank_rows", "moe_dispatch_dedup",
    "moe_expand_dedup", "moe_status_string", "moe_plan_layout", "moe_plan_dispatch_ws",
    "moe_plan_layout_dispatch", "moe_plan_combine", "moe_plan_layout_ws", "moe_plan_dispatch_planned", "moe_plan_run",
)

# include/moe_probe.h: bandwidth probes for the measurement, not part of the path
PROBES = ("moe_probe_fill", "moe_probe_read", "moe_probe_copy")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python combine_moe_layout_02_amd/build.py` "
            "(hipcc, gfx950). There is no fallback implementation."
        )
    lib = ctypes.CDLL(_LIB_PATH)
    missing = [name for name in EXPORTED + PROBES if not hasattr(lib, name)]
    if missing:
        raise ImportError(f"{_LIB_PATH} is stale (missing {missing}); rebuild it with "
                          "`python combine_moe_layout_02_amd/build.py`")
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "moe_slot_bytes": (I64, [I32]),
        "moe_window_bytes": (I64, [I32, I32, I32]),
        "moe_slot_offsets": (ctypes.c_int, [I32, I32, P, P, P, P]),
        "moe_layout": (ctypes.c_int, [P, I32, I32, I32, I32, I32] + [P] * 9 + [P]),
        "moe_layout_ex": (ctypes.c_int, [P, I32, I32, I32, I32, I32] + [P] * 9 + [I32, P]),
        "moe_dispatch": (ctypes.c_int, [P, P, I32, I32, I32, I32, I32, P, I64, P]),
        "moe_dispatch_workspace_bytes": (I64, [I32, I32, I32]),
        "moe_dispatch_ws": (ctypes.c_int, [P, P, I32, I32, I32, I32, I32, P, I64, P, I64, P]),
        "moe_dispatch_noalloc": (ctypes.c_int, [P, P, I32, I32, I32, I32, I32, P, I64, P]),
        "moe_layout_dispatch": (ctypes.c_int, [P, I32, I32, I32, I32, I32] + [P] * 9 +
                                [P, I32, I32, I32, P, I64, P]),
        "moe_layout_dispatch_ex": (ctypes.c_int, [P, I32, I32, I32, I32, I32] + [P] * 9 +
                                   [P, I32, I32, I32, P, I64, I32, P]),
        "moe_layout_dispatch_workspace_bytes": (I64, [I32, I32, I32, I32, I32, I32, I32]),
        "moe_layout_ws": (ctypes.c_int, [P, I32, I32, I32, I32, I32] + [P] * 9 + [I32, I32, P, I64, P]),
        "moe_dispatch_planned": (ctypes.c_int, [P, P, I32, I32, I32, I32, I32, I32, P, I64, P, I64, P]),
        "moe_layout_dispatch_ws": (ctypes.c_int, [P, I32, I32, I32, I32, I32] + [P] * 9 +
                                   [P, I32, I32, I32, P, I64, I32, P, I64, P]),
        "moe_combine": (ctypes.c_int, [P, I64, I64, P, P, I32, I32, I32, P, P]),
        "moe_combine_scatter": (ctypes.c_int, [P, I64, I64, P, P, I32, I32, I32, P, I64, I64, P]),
        "moe_combine_staged": (ctypes.c_int, [P, I64, I64, P, P, I32, I32, I32, P, P]),
        "moe_unpack": (ctypes.c_int, [P, I64, P, I32, I32, I32, I32, P, P, P, P]),
        "moe_dedup_window_bytes": (I64, [I32, I32, I32, I32]),
        "moe_rank_rows": (ctypes.c_int, [P, I32, I32, I32, I32, I32, P, P, P, P, P]),
        "moe_dispatch_dedup": (ctypes.c_int, [P, P, P, I32, I32, I32, I32, I32, I32, I32, P, I64, P]),
        "moe_expand_dedup": (ctypes.c_int, [P, I64, P, P, P, I32, I32, I32, I32, I32, P, P, P, P]),
        "moe_unpack_padded": (ctypes.c_int, [P, I64, P, I32, I32, I32, I32, I32, I32, I64,
                                             P, P, P, P, P, P]),
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_plan_layout": (ctypes.c_int, [P, P, I32, I32, I32, I32, I32] + [P] * 9 + [I32]),
        "moe_plan_dispatch_ws": (ctypes.c_int, [P, P, P, I32, I32, I32, I32, I32, P, I64, P, I64]),
        "moe_plan_layout_ws": (ctypes.c_int, [P, P, I32, I32, I32, I32, I32] + [P] * 9 + [I32, I32, P, I64]),
        "moe_plan_dispatch_planned": (ctypes.c_int, [P, P, P, I32, I32, I32, I32, I32, I32, P, I64, P, I64]),
        "moe_plan_layout_dispatch": (ctypes.c_int, [P, P, I32, I32, I32, I32, I32] + [P] * 9 +
                                     [P, I32, I32, I32, P, I64, I32]),
        "moe_plan_combine": (ctypes.c_int, [P, P, I64, I64, P, P, I32, I32, I32, P]),
        "moe_plan_run": (ctypes.c_int, [P, P]),
        "moe_probe_fill": (ctypes.c_int, [P, I64, P]),
        "moe_probe_read": (ctypes.c_int, [P, I64, P, P]),
        "moe_probe_copy": (ctypes.c_int, [P, P, I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


class MoeError(RuntimeError):
    """A HIP launch error reported by the library."""


def moe_status_string(status):
    return _lib.moe_status_string(int(status)).decode()


def _check(status):
    if status == MOE_OK:
        return
    msg = f"{moe_status_string(status)} (status {status})"
    if status == MOE_ERR_HIP:
        raise MoeError(msg)
    raise ValueError(msg)


# The raw handle of the current stream without building a torch Stream object (about 2 us per
# call less); torch.cuda.current_stream is the fallback where that accessor is missing.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if _raw_stream is not None:
        return _raw_stream(dev.index if dev.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return t.data_ptr()


def _need(t, name, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_layout(out, S, K, E, P, C, dev):
    """The nine Layout buffers: device, dtype, shape and contiguity."""
    shapes = ((S, P), (P,), (E,), (P, C), (E, C), (P + 1,), (E + 1,), (S, K), (1,))
    for i, (t, shp) in enumerate(zip(out, shapes)):
        dtype = torch.bool if i == 0 else torch.int32
        if (not isinstance(t, torch.Tensor) or t.device != dev or t.dtype != dtype
                or t.shape != shp or not t.is_contiguous()):
            name = Layout._fields[i]
            _need(t, name, dtype, device=dev)
            raise ValueError(f"{name} must have shape {shp}, got {tuple(t.shape)}")


def moe_slot_bytes(H):
    v = _lib.moe_slot_bytes(int(H))
    if v < 0:
        _check(int(v))
    return int(v)


def moe_window_bytes(S, K, H):
    v = _lib.moe_window_bytes(int(S), int(K), int(H))
    if v < 0:
        _check(int(v))
    return int(v)


def moe_slot_offsets(H, quant=MOE_QUANT_NONE):
    vals = [ctypes.c_int64() for _ in range(4)]
    _check(_lib.moe_slot_offsets(int(H), int(quant), *[ctypes.byref(v) for v in vals]))
    keys = ("payload_bytes", "scale_off", "triple_off", "tail_end")
    return {k: v.value for k, v in zip(keys, vals)}


class Layout(NamedTuple):
    is_token_in_rank: torch.Tensor  # bool [S, P]
    num_tokens_per_rank: torch.Tensor  # int32 [P]
    num_tokens_per_expert: torch.Tensor  # int32 [E]
    rank_prefix_matrix: torch.Tensor  # int32 [P, C]
    expert_prefix_matrix: torch.Tensor  # int32 [E, C]
    rank_slot_base: torch.Tensor  # int32 [P + 1]
    expert_slot_base: torch.Tensor  # int32 [E + 1]
    slot_idx: torch.Tensor  # int32 [S, K]
    status: torch.Tensor  # int32 [1]


def empty_layout(S, K, E, P, C, device):
    """Output buffers for moe_layout (allocation only)."""
    i32 = dict(dtype=torch.int32, device=device)
    return Layout(
        torch.empty((S, P), dtype=torch.bool, device=device),
        torch.empty(P, **i32), torch.empty(E, **i32), torch.empty((P, C), **i32),
        torch.empty((E, C), **i32), torch.empty(P + 1, **i32), torch.empty(E + 1, **i32),
        torch.empty((S, K), **i32), torch.empty(1, **i32),
    )


def moe_layout(topk_idx, num_experts, num_ranks, num_channels, out=None, stream=None, path=None):
    """Routing layout of topk_idx (int32 [S, K]) for E experts over P ranks and C channels.
    path: None (moe_layout: the form is chosen by size) or a MOE_LAYOUT_* value (moe_layout_ex)."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    S, K = topk_idx.shape
    E, P, C = int(num_experts), int(num_ranks), int(num_channels)
    dev = topk_idx.device
    if out is None:
        out = empty_layout(S, K, E, P, C, dev)
    _need_layout(out, S, K, E, P, C, dev)
    if path is None:
        _check(_lib.moe_layout(_ptr(topk_idx), S, K, E, P, C, *[_ptr(t) for t in out],
                               _stream(dev, stream)))
    else:
        _check(_lib.moe_layout_ex(_ptr(topk_idx), S, K, E, P, C, *[_ptr(t) for t in out], int(path),
                                  _stream(dev, stream)))
    return out


def moe_dispatch(x, slot_idx, window, quant=MOE_QUANT_NONE, src_rank=0, stream=None):
    """Pack bf16 rows x [S, H] into the window slots named by slot_idx [S, K]."""
    _need(x, "x", torch.bfloat16, 2)
    _need(slot_idx, "slot_idx", torch.int32, 2, x.device)
    _need(window, "window", device=x.device)
    S, H = x.shape
    if slot_idx.shape[0] != S:
        raise ValueError("slot_idx must have one row per token of x")
    K = slot_idx.shape[1]
    nbytes = window.numel() * window.element_size()
    _check(_lib.moe_dispatch(_ptr(x), _ptr(slot_idx), S, H, K, int(quant), int(src_rank),
                             _ptr(window), nbytes, _stream(x.device, stream)))
    return window


def moe_dispatch_workspace_bytes(S, K, quant=MOE_QUANT_NONE):
    v = _lib.moe_dispatch_workspace_bytes(int(S), int(K), int(quant))
    if v < 0:
        _check(int(v))
    return int(v)


def moe_dispatch_ws(x, slot_idx, window, workspace, quant=MOE_QUANT_NONE, src_rank=0, stream=None):
    """moe_dispatch with a caller workspace (a device buffer of at least
    moe_dispatch_workspace_bytes(S, K, quant) bytes, or None when that size is 0): the same window
    bytes, written by the planned pack where it applies."""
    _need(x, "x", torch.bfloat16, 2)
    _need(slot_idx, "slot_idx", torch.int32, 2, x.device)
    _need(window, "window", device=x.device)
    S, H = x.shape
    if slot_idx.shape[0] != S:
        raise ValueError("slot_idx must have one row per token of x")
    K = slot_idx.shape[1]
    if workspace is None:
        ws_ptr, ws_bytes = None, 0
    else:
        _need(workspace, "workspace", device=x.device)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    nbytes = window.numel() * window.element_size()
    _check(_lib.moe_dispatch_ws(_ptr(x), _ptr(slot_idx), S, H, K, int(quant), int(src_rank), _ptr(window),
                                nbytes, ws_ptr, ws_bytes, _stream(x.device, stream)))
    return window


def moe_dispatch_noalloc(x, slot_idx, window, quant=MOE_QUANT_NONE, src_rank=0, stream=None):
    """moe_dispatch_ws with the library's fixed device scratch instead of a workspace (allocates
    nothing; calls that overlap on one GPU race on that scratch). ValueError with MOE_ERR_SCRATCH
    when the table needs more than MOE_NOALLOC_SCRATCH_BYTES."""
    _need(x, "x", torch.bfloat16, 2)
    _need(slot_idx, "slot_idx", torch.int32, 2, x.device)
    _need(window, "window", device=x.device)
    S, H = x.shape
    if slot_idx.shape[0] != S:
        raise ValueError("slot_idx must have one row per token of x")
    K = slot_idx.shape[1]
    nbytes = window.numel() * window.element_size()
    _check(_lib.moe_dispatch_noalloc(_ptr(x), _ptr(slot_idx), S, H, K, int(quant), int(src_rank), _ptr(window),
                                     nbytes, _stream(x.device, stream)))
    return window


def moe_layout_dispatch(topk_idx, num_experts, num_ranks, num_channels, x, window,
                        quant=MOE_QUANT_NONE, src_rank=0, out=None, stream=None, path=None):
    """moe_layout and moe_dispatch in one call (one kernel for small tables); returns the Layout.
    path: None (moe_layout_dispatch) or a MOE_LAYOUT_* value (moe_layout_dispatch_ex)."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    dev = topk_idx.device
    _need(x, "x", torch.bfloat16, 2, dev)
    _need(window, "window", device=dev)
    S, K = topk_idx.shape
    if x.shape[0] != S:
        raise ValueError("x must have one row per token of topk_idx")
    H = x.shape[1]
    E, P, C = int(num_experts), int(num_ranks), int(num_channels)
    if out is None:
        out = empty_layout(S, K, E, P, C, dev)
    _need_layout(out, S, K, E, P, C, dev)
    nbytes = window.numel() * window.element_size()
    if path is None:
        _check(_lib.moe_layout_dispatch(_ptr(topk_idx), S, K, E, P, C, *[_ptr(t) for t in out],
                                        _ptr(x), H, int(quant), int(src_rank), _ptr(window), nbytes,
                                        _stream(dev, stream)))
    else:
        _check(_lib.moe_layout_dispatch_ex(_ptr(topk_idx), S, K, E, P, C, *[_ptr(t) for t in out],
                                           _ptr(x), H, int(quant), int(src_rank), _ptr(window), nbytes,
                                           int(path), _stream(dev, stream)))
    return out


def moe_layout_dispatch_workspace_bytes(S, K, E, P, C, quant=MOE_QUANT_NONE, path=MOE_LAYOUT_AUTO):
    v = _lib.moe_layout_dispatch_workspace_bytes(int(S), int(K), int(E), int(P), int(C), int(quant), int(path))
    if v < 0:
        _check(int(v))
    return int(v)


def _ws_arg(workspace, dev):
    if workspace is None:
        return None, 0
    _need(workspace, "workspace", device=dev)
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def moe_layout_ws(topk_idx, num_experts, num_ranks, num_channels, workspace, quant=MOE_QUANT_NONE,
                  out=None, stream=None, path=MOE_LAYOUT_AUTO):
    """moe_layout with a caller workspace (moe_layout_dispatch_workspace_bytes(...) bytes, or None when
    that is 0): two kernels, and in bf16 the pack plan for moe_dispatch_planned."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    dev = topk_idx.device
    S, K = topk_idx.shape
    E, P, C = int(num_experts), int(num_ranks), int(num_channels)
    if out is None:
        out = empty_layout(S, K, E, P, C, dev)
    _need_layout(out, S, K, E, P, C, dev)
    ws_ptr, ws_bytes = _ws_arg(workspace, dev)
    _check(_lib.moe_layout_ws(_ptr(topk_idx), S, K, E, P, C, *[_ptr(t) for t in out], int(quant), int(path),
                              ws_ptr, ws_bytes, _stream(dev, stream)))
    return out


def moe_dispatch_planned(x, slot_idx, window, workspace, num_channels, quant=MOE_QUANT_NONE, src_rank=0,
                         stream=None):
    """The pack of the table moe_layout_ws just laid out, from the plan it left in `workspace`."""
    _need(x, "x", torch.bfloat16, 2)
    dev = x.device
    _need(slot_idx, "slot_idx", torch.int32, 2, dev)
    _need(window, "window", device=dev)
    S, H = x.shape
    if slot_idx.shape[0] != S:
        raise ValueError("slot_idx must have one row per token of x")
    K = slot_idx.shape[1]
    ws_ptr, ws_bytes = _ws_arg(workspace, dev)
    nbytes = window.numel() * window.element_size()
    _check(_lib.moe_dispatch_planned(_ptr(x), _ptr(slot_idx), S, H, K, int(num_channels), int(quant),
                                     int(src_rank), _ptr(window), nbytes, ws_ptr, ws_bytes, _stream(dev, stream)))
    return window


def moe_layout_dispatch_ws(topk_idx, num_experts, num_ranks, num_channels, x, window, workspace,
                           quant=MOE_QUANT_NONE, src_rank=0, out=None, stream=None, path=MOE_LAYOUT_AUTO):
    """moe_layout_dispatch with a caller workspace (at least moe_layout_dispatch_workspace_bytes(...)
    bytes, or None when that size is 0): two layout kernels, the pack plan written by the layout."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    dev = topk_idx.device
    _need(x, "x", torch.bfloat16, 2, dev)
    _need(window, "window", device=dev)
    S, K = topk_idx.shape
    if x.shape[0] != S:
        raise ValueError("x must have one row per token of topk_idx")
    H = x.shape[1]
    E, P, C = int(num_experts), int(num_ranks), int(num_channels)
    if out is None:
        out = empty_layout(S, K, E, P, C, dev)
    _need_layout(out, S, K, E, P, C, dev)
    ws_ptr, ws_bytes = _ws_arg(workspace, dev)
    nbytes = window.numel() * window.element_size()
    _check(_lib.moe_layout_dispatch_ws(_ptr(topk_idx), S, K, E, P, C, *[_ptr(t) for t in out], _ptr(x), H,
                                       int(quant), int(src_rank), _ptr(window), nbytes, int(path), ws_ptr,
                                       ws_bytes, _stream(dev, stream)))
    return out


def moe_combine(expert_out, slot_idx, topk_weights, row_stride_bytes=None, expert_rows=None,
                hidden=None, y=None, stream=None):
    """y[t] = bf16(sum_k w[t,k] * expert_out[slot_idx[t,k]]) with fp32 accumulation.

    expert_out is either a bf16 [R, H] tensor (row stride 2H, R rows) or any device
    buffer with explicit row_stride_bytes, expert_rows and hidden (for example the
    dispatch window with row_stride_bytes = moe_slot_bytes(H)).
    """
    _need(slot_idx, "slot_idx", torch.int32, 2)
    dev = slot_idx.device
    _need(expert_out, "expert_out", device=dev)
    _need(topk_weights, "topk_weights", torch.float32, 2, dev)
    S, K = slot_idx.shape
    if tuple(topk_weights.shape) != (S, K):
        raise ValueError("topk_weights must match slot_idx")
    if row_stride_bytes is None:
        if expert_out.dtype != torch.bfloat16 or expert_out.dim() != 2:
            raise ValueError("pass row_stride_bytes/expert_rows/hidden for a non-[R, H] bf16 buffer")
        expert_rows, H = expert_out.shape
        row_stride_bytes = 2 * H
    else:
        if expert_rows is None or hidden is None:
            raise ValueError("expert_rows and hidden are required with row_stride_bytes")
        H = int(hidden)
        if int(expert_rows) * int(row_stride_bytes) > expert_out.numel() * expert_out.element_size():
            raise ValueError("expert_rows * row_stride_bytes exceeds the expert_out buffer")
    if y is None:
        y = torch.empty((S, H), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, 2, dev)
    if tuple(y.shape) != (S, H):
        raise ValueError(f"y must have shape {(S, H)}")
    _check(_lib.moe_combine(_ptr(expert_out), int(row_stride_bytes), int(expert_rows),
                            _ptr(slot_idx), _ptr(topk_weights), S, H, K, _ptr(y),
                            _stream(dev, stream)))
    return y


def moe_combine_scatter(expert_out, expand_idx, num_rows, S, K, staging=None, staging_stride_bytes=None,
                        stream=None):
    """First pass of the two-pass combine: bf16 expert rows [R, H] (row s for slot s) to staging
    row t*K + k by their triples expand_idx [R, 3]; rows at or past the device count num_rows are
    skipped. staging defaults to a new bf16 [S*K, H] tensor (stride 2H)."""
    _need(expert_out, "expert_out", torch.bfloat16, 2)
    dev = expert_out.device
    _need(expand_idx, "expand_idx", torch.int32, 2, dev)
    _need(num_rows, "num_rows", torch.int32, device=dev)
    R, H = expert_out.shape
    S, K = int(S), int(K)
    if tuple(expand_idx.shape) != (R, 3):
        raise ValueError("expand_idx must be [rows of expert_out, 3]")
    if staging is None:
        staging = torch.empty((S * K, H), dtype=torch.bfloat16, device=dev)
    _need(staging, "staging", device=dev)
    stride = 2 * H if staging_stride_bytes is None else int(staging_stride_bytes)
    _check(_lib.moe_combine_scatter(_ptr(expert_out), 2 * H, R, _ptr(expand_idx), _ptr(num_rows), S, K,
                                    H, _ptr(staging), stride, staging.numel() * staging.element_size(),
                                    _stream(dev, stream)))
    return staging


def moe_combine_staged(staging, slot_idx, topk_weights, hidden, staging_stride_bytes=None, y=None,
                       stream=None):
    """Second pass of the two-pass combine: y[t] reduces staging rows t*K .. t*K+K-1 (entries with
    slot_idx < 0 skipped) with the arithmetic of moe_combine."""
    _need(slot_idx, "slot_idx", torch.int32, 2)
    dev = slot_idx.device
    _need(staging, "staging", device=dev)
    _need(topk_weights, "topk_weights", torch.float32, 2, dev)
    S, K = slot_idx.shape
    H = int(hidden)
    stride = 2 * H if staging_stride_bytes is None else int(staging_stride_bytes)
    if tuple(topk_weights.shape) != (S, K):
        raise ValueError("topk_weights must match slot_idx")
    if y is None:
        y = torch.empty((S, H), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, 2, dev)
    if tuple(y.shape) != (S, H):
        raise ValueError(f"y must have shape {(S, H)}")
    _check(_lib.moe_combine_staged(_ptr(staging), stride, staging.numel() * staging.element_size(),
                                   _ptr(slot_idx), _ptr(topk_weights), S, H, K, _ptr(y),
                                   _stream(dev, stream)))
    return y


def moe_probe_fill(dst, stream=None):
    """Write-only bandwidth probe over the whole device tensor dst (measurement only)."""
    _need(dst, "dst")
    _check(_lib.moe_probe_fill(_ptr(dst), dst.numel() * dst.element_size(), _stream(dst.device, stream)))


def moe_probe_read(src, sink, stream=None):
    """Read-only bandwidth probe over the whole device tensor src; sink is a device int32 [1]."""
    _need(src, "src")
    _need(sink, "sink", torch.int32, device=src.device)
    _check(_lib.moe_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                               _stream(src.device, stream)))


def moe_probe_copy(src, dst, stream=None):
    """Copy probe: dst = src, both device tensors of the same byte size."""
    _need(src, "src")
    _need(dst, "dst", device=src.device)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst must have the same byte size")
    _check(_lib.moe_probe_copy(_ptr(src), _ptr(dst), n, _stream(src.device, stream)))


MOE_PLAN_BYTES = 320  # sizeof(moe_plan)


class Plan:
    """A pre-validated call (include/moe.h, moe_plan_*): the arguments were checked once when the
    plan was made; run() enqueues the call on the current (or given) stream without checking them
    again. The tensors the plan was made from are kept referenced here, so they stay allocated for
    the plan's lifetime; they must keep their shapes (do not resize them)."""

    __slots__ = ("_buf", "_addr", "_dev", "_keep", "_run", "_stream_of")

    def __init__(self, dev, keep):
        self._buf = ctypes.create_string_buffer(MOE_PLAN_BYTES)
        self._addr = ctypes.addressof(self._buf)
        self._dev = dev.index if dev.index is not None else torch.cuda.current_device()
        self._keep = keep
        self._run = _lib.moe_plan_run
        self._stream_of = _raw_stream

    def run(self, stream=None):
        if stream is None and self._stream_of is not None:
            rc = self._run(self._addr, self._stream_of(self._dev))
        else:
            rc = self._run(self._addr, _stream(torch.device("cuda", self._dev), stream))
        if rc:
            _check(rc)


def plan_layout(topk_idx, num_experts, num_ranks, num_channels, out, path=MOE_LAYOUT_AUTO):
    """Plan of moe_layout_ex on these buffers (out: a Layout)."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    S, K = topk_idx.shape
    E, P, C = int(num_experts), int(num_ranks), int(num_channels)
    dev = topk_idx.device
    _need_layout(out, S, K, E, P, C, dev)
    plan = Plan(dev, (topk_idx, out))
    _check(_lib.moe_plan_layout(plan._addr, _ptr(topk_idx), S, K, E, P, C, *[_ptr(t) for t in out], int(path)))
    return plan


def plan_dispatch_ws(x, slot_idx, window, workspace, quant=MOE_QUANT_NONE, src_rank=0):
    """Plan of moe_dispatch_ws on these buffers."""
    _need(x, "x", torch.bfloat16, 2)
    _need(slot_idx, "slot_idx", torch.int32, 2, x.device)
    _need(window, "window", device=x.device)
    S, H = x.shape
    if slot_idx.shape[0] != S:
        raise ValueError("slot_idx must have one row per token of x")
    K = slot_idx.shape[1]
    if workspace is None:
        ws_ptr, ws_bytes = None, 0
    else:
        _need(workspace, "workspace", device=x.device)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    plan = Plan(x.device, (x, slot_idx, window, workspace))
    _check(_lib.moe_plan_dispatch_ws(plan._addr, _ptr(x), _ptr(slot_idx), S, H, K, int(quant), int(src_rank),
                                     _ptr(window), window.numel() * window.element_size(), ws_ptr, ws_bytes))
    return plan


def plan_layout_ws(topk_idx, num_experts, num_ranks, num_channels, out, workspace, quant=MOE_QUANT_NONE,
                   path=MOE_LAYOUT_AUTO):
    """Plan of moe_layout_ws on these buffers (out: a Layout)."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    S, K = topk_idx.shape
    E, P, C = int(num_experts), int(num_ranks), int(num_channels)
    dev = topk_idx.device
    _need_layout(out, S, K, E, P, C, dev)
    ws_ptr, ws_bytes = _ws_arg(workspace, dev)
    plan = Plan(dev, (topk_idx, out, workspace))
    _check(_lib.moe_plan_layout_ws(plan._addr, _ptr(topk_idx), S, K, E, P, C, *[_ptr(t) for t in out], int(quant),
                                   int(path), ws_ptr, ws_bytes))
    return plan


def plan_dispatch_planned(x, slot_idx, window, workspace, num_channels, quant=MOE_QUANT_NONE, src_rank=0):
    """Plan of moe_dispatch_planned on these buffers."""
    _need(x, "x", torch.bfloat16, 2)
    _need(slot_idx, "slot_idx", torch.int32, 2, x.device)
    _need(window, "window", device=x.device)
    S, H = x.shape
    if slot_idx.shape[0] != S:
        raise ValueError("slot_idx must have one row per token of x")
    K = slot_idx.shape[1]
    ws_ptr, ws_bytes = _ws_arg(workspace, x.device)
    plan = Plan(x.device, (x, slot_idx, window, workspace))
    _check(_lib.moe_plan_dispatch_planned(plan._addr, _ptr(x), _ptr(slot_idx), S, H, K, int(num_channels), int(quant),
                                          int(src_rank), _ptr(window), window.numel() * window.element_size(),
                                          ws_ptr, ws_bytes))
    return plan


def plan_layout_dispatch(topk_idx, num_experts, num_ranks, num_channels, x, window, out, quant=MOE_QUANT_NONE,
                         src_rank=0, path=MOE_LAYOUT_AUTO):
    """Plan of moe_layout_dispatch_ex on these buffers (out: a Layout)."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    dev = topk_idx.device
    _need(x, "x", torch.bfloat16, 2, dev)
    _need(window, "window", device=dev)
    S, K = topk_idx.shape
    if x.shape[0] != S:
        raise ValueError("x must have one row per token of topk_idx")
    E, P, C = int(num_experts), int(num_ranks), int(num_channels)
    _need_layout(out, S, K, E, P, C, dev)
    plan = Plan(dev, (topk_idx, x, window, out))
    _check(_lib.moe_plan_layout_dispatch(plan._addr, _ptr(topk_idx), S, K, E, P, C, *[_ptr(t) for t in out],
                                         _ptr(x), x.shape[1], int(quant), int(src_rank), _ptr(window),
                                         window.numel() * window.element_size(), int(path)))
    return plan


def plan_combine(expert_out, slot_idx, topk_weights, y):
    """Plan of moe_combine of a bf16 [R, H] expert_out into y (bf16 [S, H])."""
    _need(slot_idx, "slot_idx", torch.int32, 2)
    dev = slot_idx.device
    _need(expert_out, "expert_out", torch.bfloat16, 2, dev)
    _need(topk_weights, "topk_weights", torch.float32, 2, dev)
    _need(y, "y", torch.bfloat16, 2, dev)
    S, K = slot_idx.shape
    R, H = expert_out.shape
    if tuple(topk_weights.shape) != (S, K) or tuple(y.shape) != (S, H):
        raise ValueError("topk_weights must match slot_idx and y must be [S, H]")
    plan = Plan(dev, (expert_out, slot_idx, topk_weights, y))
    _check(_lib.moe_plan_combine(plan._addr, _ptr(expert_out), 2 * H, R, _ptr(slot_idx), _ptr(topk_weights), S, H,
                                 K, _ptr(y)))
    return plan


def moe_dedup_window_bytes(S, K, P, H):
    v = _lib.moe_dedup_window_bytes(int(S), int(K), int(P), int(H))
    if v < 0:
        _check(int(v))
    return int(v)


class RankRows(NamedTuple):
    rank_row_idx: torch.Tensor  # int32 [S, K]
    rank_token_base: torch.Tensor  # int32 [P + 1]


def moe_rank_rows(topk_idx, layout, num_experts, num_ranks, num_channels, out=None, stream=None):
    """Per-rank deduplicated rows of the routing table, from moe_layout's rank_prefix_matrix and
    num_tokens_per_rank (layout is the Layout moe_layout returned)."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    dev = topk_idx.device
    S, K = topk_idx.shape
    E, P, C = int(num_experts), int(num_ranks), int(num_channels)
    _need(layout.rank_prefix_matrix, "rank_prefix_matrix", torch.int32, 2, dev)
    _need(layout.num_tokens_per_rank, "num_tokens_per_rank", torch.int32, 1, dev)
    if tuple(layout.rank_prefix_matrix.shape) != (P, C) or layout.num_tokens_per_rank.shape[0] != P:
        raise ValueError("layout does not match num_ranks / num_channels")
    if out is None:
        out = RankRows(torch.empty((S, K), dtype=torch.int32, device=dev),
                       torch.empty(P + 1, dtype=torch.int32, device=dev))
    _need(out.rank_row_idx, "rank_row_idx", torch.int32, 2, dev)
    _need(out.rank_token_base, "rank_token_base", torch.int32, 1, dev)
    if tuple(out.rank_row_idx.shape) != (S, K) or out.rank_token_base.shape[0] != P + 1:
        raise ValueError("rank_row_idx must be [S, K] and rank_token_base [P + 1]")
    _check(_lib.moe_rank_rows(_ptr(topk_idx), S, K, E, P, C, _ptr(layout.rank_prefix_matrix),
                              _ptr(layout.num_tokens_per_rank), _ptr(out.rank_row_idx),
                              _ptr(out.rank_token_base), _stream(dev, stream)))
    return out


def moe_dispatch_dedup(x, rank_row_idx, topk_idx, num_experts, num_ranks, window, quant=MOE_QUANT_NONE,
                       src_rank=0, stream=None):
    """One row per (token, destination rank) into the rows named by rank_row_idx (bf16, or the
    token's dynamic fp8 / INT8 codes and scale)."""
    _need(x, "x", torch.bfloat16, 2)
    dev = x.device
    _need(rank_row_idx, "rank_row_idx", torch.int32, 2, dev)
    _need(topk_idx, "topk_idx", torch.int32, 2, dev)
    _need(window, "window", device=dev)
    S, H = x.shape
    K = topk_idx.shape[1]
    if tuple(topk_idx.shape) != (S, K) or tuple(rank_row_idx.shape) != (S, K):
        raise ValueError("rank_row_idx and topk_idx must be [S, K] with S rows of x")
    nbytes = window.numel() * window.element_size()
    _check(_lib.moe_dispatch_dedup(_ptr(x), _ptr(rank_row_idx), _ptr(topk_idx), S, H, K,
                                   int(num_experts), int(num_ranks), int(quant), int(src_rank),
                                   _ptr(window), nbytes, _stream(dev, stream)))
    return window


def moe_expand_dedup(window, rank_row_idx, slot_idx, num_slots, num_ranks, H, quant=MOE_QUANT_NONE,
                     out=None, stream=None):
    """Receive-side expansion of the deduplicated rows to the expert-major rows of slot_idx:
    returns Unpacked(expand_x [S*K, H] bf16 or uint8 codes, expand_scales fp32 [S*K] or None,
    expand_idx int32 [S*K, 3]) as moe_unpack would. num_slots is the device count N
    (layout.expert_slot_base[E:])."""
    _need(window, "window")
    dev = window.device
    _need(rank_row_idx, "rank_row_idx", torch.int32, 2, dev)
    _need(slot_idx, "slot_idx", torch.int32, 2, dev)
    _need(num_slots, "num_slots", torch.int32, device=dev)
    S, K = slot_idx.shape
    H, quant = int(H), int(quant)
    rows = S * K
    if tuple(rank_row_idx.shape) != (S, K):
        raise ValueError("rank_row_idx must match slot_idx")
    if out is None:
        if quant == MOE_QUANT_NONE:
            ex, sc = torch.empty((rows, H), dtype=torch.bfloat16, device=dev), None
        else:
            ex = torch.empty((rows, H), dtype=torch.uint8, device=dev)
            sc = torch.empty(rows, dtype=torch.float32, device=dev)
        out = Unpacked(ex, sc, torch.empty((rows, 3), dtype=torch.int32, device=dev))
    ex, sc, idx = out
    _need(ex, "expand_x", device=dev)
    _need(idx, "expand_idx", torch.int32, 2, dev)
    payload = moe_slot_offsets(H, quant)["payload_bytes"]
    if ex.numel() * ex.element_size() < rows * payload or tuple(idx.shape) != (rows, 3):
        raise ValueError("expand_x must hold S*K rows of payload bytes and expand_idx [S*K, 3]")
    if sc is not None:
        _need(sc, "expand_scales", torch.float32, device=dev)
        if sc.numel() < rows:
            raise ValueError("expand_scales must hold S*K values")
    nbytes = window.numel() * window.element_size()
    _check(_lib.moe_expand_dedup(_ptr(window), nbytes, _ptr(rank_row_idx), _ptr(slot_idx),
                                 _ptr(num_slots), S, K, int(num_ranks), H, quant, _ptr(ex),
                                 None if sc is None else _ptr(sc), _ptr(idx), _stream(dev, stream)))
    return out


class Unpacked(NamedTuple):
    expand_x: torch.Tensor  # [S*K, H] bf16, or uint8 codes for the quantised modes
    expand_scales: torch.Tensor  # fp32 [S*K] (quantised modes) or None
    expand_idx: torch.Tensor  # int32 [S*K, 3]


def moe_unpack(window, num_slots, S, K, H, quant=MOE_QUANT_NONE, out=None, stream=None):
    """Compact rows, triples and scales of the first N window slots (N read on the device from
    num_slots, e.g. layout.expert_slot_base[E:]). Rows N..S*K-1 of the outputs are left as is."""
    _need(window, "window")
    dev = window.device
    _need(num_slots, "num_slots", torch.int32, device=dev)
    S, K, H, quant = int(S), int(K), int(H), int(quant)
    rows = S * K
    if out is None:
        if quant == MOE_QUANT_NONE:
            ex = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
            sc = None
        else:
            ex = torch.empty((rows, H), dtype=torch.uint8, device=dev)
            sc = torch.empty(rows, dtype=torch.float32, device=dev)
        out = Unpacked(ex, sc, torch.empty((rows, 3), dtype=torch.int32, device=dev))
    ex, sc, idx = out
    _need(ex, "expand_x", device=dev)
    _need(idx, "expand_idx", torch.int32, 2, dev)
    payload = moe_slot_offsets(H, quant)["payload_bytes"]
    if ex.numel() * ex.element_size() < rows * payload or tuple(idx.shape) != (rows, 3):
        raise ValueError("expand_x must hold S*K rows of payload bytes and expand_idx [S*K, 3]")
    if sc is not None:
        _need(sc, "expand_scales", torch.float32, device=dev)
        if sc.numel() < rows:
            raise ValueError("expand_scales must hold S*K values")
    nbytes = window.numel() * window.element_size()
    _check(_lib.moe_unpack(_ptr(window), nbytes, _ptr(num_slots), S, K, H, quant, _ptr(ex),
                           None if sc is None else _ptr(sc), _ptr(idx), _stream(dev, stream)))
    return out


class PaddedUnpacked(NamedTuple):
    expand_x: torch.Tensor  # [R, H] bf16, or uint8 codes for the quantised modes
    expand_scales: torch.Tensor  # fp32 [R] (quantised modes) or None
    expand_idx: torch.Tensor  # int32 [R, 3], (-1, -1, -1) on padding rows
    expert_row_base: torch.Tensor  # int32 [E + 1], aligned first row of each expert
    status: torch.Tensor  # int32 [1], 1 if the aligned rows exceeded R


def moe_unpack_padded(window, expert_slot_base, S, K, H, quant=MOE_QUANT_NONE, expert_alignment=1,
                      out_rows=None, out=None, stream=None):
    """Unpack into exactly out_rows rows (default S*K) with each expert's block starting at a
    multiple of expert_alignment; padding rows are zero with triple -1. expert_slot_base is the
    layout's device tensor [E + 1]; nothing is read back to the host."""
    _need(window, "window")
    dev = window.device
    _need(expert_slot_base, "expert_slot_base", torch.int32, 1, dev)
    S, K, H, quant = int(S), int(K), int(H), int(quant)
    E = expert_slot_base.shape[0] - 1
    R = S * K if out_rows is None else int(out_rows)
    if out is None:
        if quant == MOE_QUANT_NONE:
            ex = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
            sc = None
        else:
            ex = torch.empty((R, H), dtype=torch.uint8, device=dev)
            sc = torch.empty(R, dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        out = PaddedUnpacked(ex, sc, torch.empty((R, 3), **i32), torch.empty(E + 1, **i32),
                             torch.empty(1, **i32))
    ex, sc, idx, base, status = out
    _need(ex, "expand_x", device=dev)
    _need(idx, "expand_idx", torch.int32, 2, dev)
    _need(base, "expert_row_base", torch.int32, 1, dev)
    _need(status, "status", torch.int32, device=dev)
    payload = moe_slot_offsets(H, quant)["payload_bytes"]
    if ex.numel() * ex.element_size() < R * payload or tuple(idx.shape) != (R, 3):
        raise ValueError("expand_x must hold out_rows rows of payload bytes and expand_idx [out_rows, 3]")
    if base.shape[0] != E + 1 or status.numel() < 1:
        raise ValueError("expert_row_base must have E + 1 entries and status one")
    if sc is not None:
        _need(sc, "expand_scales", torch.float32, device=dev)
        if sc.numel() < R:
            raise ValueError("expand_scales must hold out_rows values")
    nbytes = window.numel() * window.element_size()
    _check(_lib.moe_unpack_padded(_ptr(window), nbytes, _ptr(expert_slot_base), E, S, K, H, quant,
                                  int(expert_alignment), R, _ptr(ex), None if sc is None else _ptr(sc),
                                  _ptr(idx), _ptr(base), _ptr(status), _stream(dev, stream)))
    return out


__all__ = [
    "MOE_OK", "MOE_ERR_ARG", "MOE_ERR_ALIGN", "MOE_ERR_WINDOW", "MOE_ERR_UNSUPPORTED",
    "MOE_ERR_HIP", "MOE_QUANT_NONE", "MOE_QUANT_FP8_E4M3_DYN", "MOE_QUANT_INT8_DYN", "MOE_LAYOUT_AUTO",
    "MOE_LAYOUT_MULTI", "MOE_LAYOUT_SINGLE", "MoeError", "Layout",
    "empty_layout", "moe_slot_bytes", "moe_window_bytes", "moe_slot_offsets", "moe_layout",
    "moe_dispatch", "moe_dispatch_workspace_bytes", "moe_dispatch_ws", "moe_dispatch_noalloc", "MOE_ERR_SCRATCH",
    "moe_layout_dispatch_workspace_bytes", "moe_layout_ws", "moe_dispatch_planned", "moe_layout_dispatch_ws",
    "MOE_NOALLOC_SCRATCH_BYTES", "moe_layout_dispatch", "moe_combine", "moe_combine_scatter", "moe_combine_staged", "moe_unpack", "Unpacked", "moe_unpack_padded", "PaddedUnpacked",
    "moe_dedup_window_bytes", "moe_rank_rows", "RankRows", "moe_dispatch_dedup", "moe_expand_dedup",
    "moe_status_string", "Plan", "plan_layout", "plan_dispatch_ws", "plan_layout_dispatch", "plan_combine",
    "plan_layout_ws", "plan_dispatch_planned",
    "MOE_PLAN_BYTES",
]
