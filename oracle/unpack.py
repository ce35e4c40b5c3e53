"""Unpack: window slots -> compact expert input rows, their triples and scales.

Test infrastructure only (see the package docstring).

The CAM receive side ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.9 ShareToOutput)
walks the received slots in (local expert, source rank) order and copies each slot's token data to
the next row of expandXOut and its triple (source rank, token index, k) to the same row of
expandIdxOut. On one GPU the window's slots are already in expert-major, source-token order, so
row s of the compact output is slot s: the unpack strips each slot's padding and tail. For the
quantised modes the per-row scale read from the slot's scale block goes to its own vector, since
the codes alone do not carry it.
"""

import numpy as np

from .dispatch import QUANT_NONE, slot_geometry


def unpack(regions, H, quant=QUANT_NONE):
    """regions: uint8 [N, >= tail_end] (slot s = row s, as dispatch_slots returns).

    Returns (expand_x uint8 [N, payload_bytes], expand_idx int32 [N, 3],
    expand_scales float32 [N] or None for bf16).
    """
    g = slot_geometry(H, quant)
    regions = np.ascontiguousarray(regions, dtype=np.uint8)
    n = regions.shape[0]
    expand_x = regions[:, : g.payload_bytes].copy()
    expand_idx = regions[:, g.triple_off : g.triple_off + 12].copy().view("<i4").reshape(n, 3)
    scales = None
    if quant != QUANT_NONE:
        scales = regions[:, g.scale_off : g.scale_off + 4].copy().view("<f4").reshape(n)
    return expand_x, expand_idx.astype(np.int32), scales
