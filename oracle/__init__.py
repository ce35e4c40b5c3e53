"""Plain CPU oracle for the MoE normal-mode routing layout, dispatch pack and combine.

This package is TEST INFRASTRUCTURE. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (``combine_moe_layout_02_amd``) never imports, links or runs
anything here, and this package imports nothing from the product path: the two
share no kernels, headers, helpers, tables or constants. Only numpy is used.

Every result of the method is exact (integer layout, byte movement, one defined
fp32 reduction), so each function here is the plain definition of its result,
written out step by step. Citations name the page title and the section on it:

* "HCCL Window 模式 (Non-SHMEM) 代码深度剖析" (the CAM window-mode analysis):
  section 2.3 (token slot format), 3.6 (InputToShare), 3.9 (ShareToOutput),
  7.8 (ReadBufferAndWeightedSum), 8.2 (window size check), 8.3 (core split).
* "Ascend DeepEP MoE Dispatch Optimization": "一条 token 如何走完 MoE" (token path,
  dst_rank), "Dispatch handle 六项分别保存什么" (handle tensors), "Notify 先交换数量和前缀"
  (counts and prefix sums), "Device 侧如何把 channel 变成远端 Put" (per-channel cursor),
  "所谓 compact plan 到底压缩了什么" (compact destination plan), "P 维路由为什么值得单独优化"
  (per-destination segments), "输出长度有动态和固定两种模式"
  (fixed-length num_worst_tokens outputs).
* "internode.cu", section 1 notify_dispatch (per-rank / per-expert counting, the
  expert_alignment rounding of the per-expert counts).

Where the pages leave a step open, the reading taken is stated in the function's
docstring.
"""

from .formats import (
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    e4m3fn_decode,
    e4m3fn_encode,
    E4M3FN_MAX,
)
from .layout import channel_bounds, layout, layout_bruteforce
from .dispatch import (
    slot_geometry,
    quantize_e4m3_dynamic,
    quantize_int8_dynamic,
    dispatch_slots,
    dispatch_slots_bruteforce,
)
from .combine import combine, combine_bruteforce, combine_scatter, combine_staged
from .unpack import aligned_row_base, unpack, unpack_padded
from .dedup import dispatch_dedup, expand_dedup, rank_rows

__all__ = [
    "bf16_bits_to_f32",
    "f32_to_bf16_bits",
    "e4m3fn_decode",
    "e4m3fn_encode",
    "E4M3FN_MAX",
    "channel_bounds",
    "layout",
    "layout_bruteforce",
    "slot_geometry",
    "quantize_e4m3_dynamic",
    "quantize_int8_dynamic",
    "dispatch_slots",
    "dispatch_slots_bruteforce",
    "combine",
    "combine_bruteforce",
    "combine_scatter",
    "combine_staged",
    "unpack",
    "aligned_row_base",
    "unpack_padded",
    "rank_rows",
    "dispatch_dedup",
    "expand_dedup",
]
