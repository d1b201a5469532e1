"""CPU fp64 oracle for exact attention -- TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The HIP
library never imports it and it never imports the HIP library: the two share
no kernels, headers, helpers, tables or pre/post-processing.  Inputs reach
both sides from the seeded generators in ``workloads.py``, which hold none of
the method's arithmetic.

Pages cited (titles/sections as printed on them):
  [ctyun]  ctyun.cn developer article on FlashAttention -- sections
           "背景 / Transformer的复杂度", "核心思想", "MAC分析".
  [jiahao] "Flash Attention" note on special-jiahao.github.io -- sections
           "Standard Attention", "增量求解 softmax" (also the block merge
           of partial attention results, merge.py).
  [xinc]   xinc.fun archive 235 -- sections "6. 标准注意力为什么慢",
           "7. Online Softmax" (also its closing remark on the backward
           pass, backward.py), "4. 减少访存的几种办法" (FP8 matrix-product
           inputs, fp8.py).

Every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` against something other than itself (brute
force in 40-digit decimal arithmetic, closed forms, hand-derived fixtures in
``tests/golden/``, library conversions, invariants).  No function is
"parity unpinned".
"""

from .attention import (
    decode_bf16,
    decode_f16,
    decode_f32,
    standard_attention,
    standard_attention_rows,
)
from .softmax import (
    local_softmax,
    online_row_stats,
    online_softmax_output,
    softmax_rows,
    two_block_softmax,
)
from .tiled import tiled_online_attention
from .mac_count import standard_attention_mac
from .merge import merge_partials, partial_attention
from .backward import attention_backward
from .fp8 import decode_e4m3, fp8_attention, fp8_attention_rows, fp8_values

__all__ = [
    "decode_bf16",
    "decode_f16",
    "decode_f32",
    "standard_attention",
    "standard_attention_rows",
    "local_softmax",
    "two_block_softmax",
    "online_softmax_output",
    "softmax_rows",
    "online_row_stats",
    "tiled_online_attention",
    "standard_attention_mac",
    "partial_attention",
    "merge_partials",
    "attention_backward",
    "decode_e4m3",
    "fp8_values",
    "fp8_attention",
    "fp8_attention_rows",
]
