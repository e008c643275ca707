"""Reference implementation of exact attention, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import it.  The GPU library never calls it,
shares no code with it and has no fallback to it.

Sources (the three pages the method is described on):
  * M4-047 card  - airsota.com, "高效注意力与 FlashAttention (Efficient Attention & FlashAttention)"
  * Day-21 page  - daoyuly.cn, "GPU 学习日报 Day 21：FlashAttention：GPU Memory Hierarchy 下的 IO 优化"
  * Q31 answer   - agentalpha.top, "Q31：FlashAttention 为什么快"

Modules:
  attention   - the plain definition: explicit S, two-pass safe softmax, P V, LSE;
                the per-split partials and their merge for split-KV decode.
  recurrence  - the online-softmax block recurrence in pure Python (tiny inputs only),
                used to pin the block-by-block steps against the two-pass definition.
  backward    - the gradients dQ, dK, dV by the chain rule through the same definition.
  fp8         - OCP FP8 E4M3 values and attention over FP8 inputs (KV cache; Q, K, V).

Every function here is pinned by tests marked "not gpu" (closed forms, invariants,
library special cases, brute force and the pages' own worked example).
"""
from .attention import (  # noqa: F401
    scores, softmax_two_pass, attention_head, attention, attention_probs,
    split_bounds, split_partials, combine_partials,
)
from .backward import attention_backward_head, attention_backward, softmax_row_stat  # noqa: F401
from .fp8 import e4m3_value, e4m3_decode, attention_head_fp8kv, attention_head_fp8  # noqa: F401
from . import recurrence  # noqa: F401
