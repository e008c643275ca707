"""Seeded synthetic workloads and inputs (no attention arithmetic lives here)."""
from .workloads import WORKLOADS, Workload, get, PREFILL_HEADLINE, DECODE_HEADLINE  # noqa: F401
from .inputs import (  # noqa: F401
    round_to_bf16_bits, bf16_bits_to_f32, head_block, head_block_f32, make_tensor, as_f32,
)
