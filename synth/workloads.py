"""The synthetic workloads: shapes, dtypes, masks and value recipes.

Shapes follow the workloads the pages talk about:
  * B=8, H=16, N=8192 is the batch/head/length example of the Day-21 tutorial
    ("GPU 学习日报 Day 21：FlashAttention：GPU Memory Hierarchy 下的 IO 优化", §3.2),
    where one N x N fp16 matrix already takes about 16 GB;
  * N=16384 is the length the M4-047 card ("高效注意力与 FlashAttention", §3)
    uses for its N^2 = 2.68e8 example, and the Q31 answer
    ("FlashAttention 为什么快", follow-up 1) uses for its HBM estimate;
  * Nq=1 against a long KV cache is the decode case (Day-21 tutorial §9 and FAQ Q5;
    Q31 answer follow-up 3: split K/V into chunks, compute them in parallel, merge).

This module holds no attention arithmetic.  It is shared by the tests, the
benchmark and the reference implementation's callers; nothing here depends on
the GPU library or on the reference implementation.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str  # "bf16" or "f32": storage type of Q, K, V and O
    causal: bool
    seed: int
    # Value recipe for K beyond i.i.d. N(0,1): ("none",), ("scale_all", 2.0) or
    # ("scale_rows_every", 64, 8.0) = rows j with j % 64 == 0 multiplied by 8.
    k_rule: tuple = ("none",)
    num_splits: int = 0  # > 0: decode workload, split-KV into this many partitions
    description: str = ""
    H_kv: int = 0  # K/V heads (0: H); query head h reads K/V head h // (H // H_kv)
    kv_dtype: str = ""  # "" (as dtype) or "e4m3": K and V stored as OCP FP8 E4M3 codes with a scale per
    #                     (batch, K/V head)
    q_dtype: str = ""  # "" (as dtype) or "e4m3": Q stored as E4M3 codes with a scale per (batch, head)
    causal_align: str = "top_left"  # or "bottom_right": key j visible to row i iff j <= i + Nk - Nq
    # Element mask (synth.masks): () none, ("documents", seed, min_len, max_len) packed documents
    # with causal attention inside each, ("window", w) a causal sliding window of w keys,
    # ("tiles", seed, bq, bk) random empty / full / bit-by-bit tiles of bq x bk elements
    mask_rule: tuple = ()

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def diag(self) -> int:
        return self.Nk - self.Nq if (self.causal and self.causal_align == "bottom_right") else 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def is_decode(self) -> bool:
        return self.num_splits > 0

    @property
    def elt_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            "tiny_f32_n128_d64", B=1, H=1, Nq=128, Nk=128, d=64, dtype="f32", causal=False, seed=1000,
            description="tiny reference case: fp32 Q/K/V, O[128x64] and per-row LSE"),
        Workload(
            "batch_b4h16_n2048_d64", B=4, H=16, Nq=2048, Nk=2048, d=64, dtype="bf16", causal=False,
            seed=2000, description="short-sequence batch, non-causal"),
        Workload(
            "prefill_b8h16_n8192_d128_causal", B=8, H=16, Nq=8192, Nk=8192, d=128, dtype="bf16",
            causal=True, seed=3000, k_rule=("scale_all", 2.0),
            description="causal prefill, K scaled x2 to sharpen softmax rows"),
        Workload(
            "long_b1h32_n16384_d128_causal", B=1, H=32, Nq=16384, Nk=16384, d=128, dtype="bf16",
            causal=True, seed=4000, k_rule=("scale_rows_every", 64, 8.0),
            description="long-context causal prefill, every 64th key row x8 (stresses max rescaling)"),
        Workload(
            "decode_b16h32_nk32768_d128", B=16, H=32, Nq=1, Nk=32768, d=128, dtype="bf16",
            causal=False, seed=5000, num_splits=64,
            description="1-token decode against a 32768-key cache, 64-way split-KV + combine"),
        Workload(
            "chunk_prefill_b1h32kv8_nq2048_nk16384_d128", B=1, H=32, H_kv=8, Nq=2048, Nk=16384, d=128,
            dtype="bf16", causal=True, causal_align="bottom_right", seed=6000,
            description="a 2048-token prompt chunk appended to a 14336-token cache (bottom-right causal), "
                        "four query heads per K/V head"),
        Workload(
            "decode_gqa_b16h32kv8_nk32768_d128", B=16, H=32, H_kv=8, Nq=1, Nk=32768, d=128, dtype="bf16",
            causal=False, seed=7000, num_splits=64,
            description="1-token decode with four query heads per K/V head, 64-way split-KV + combine"),
        Workload(
            "decode_fp8kv_b16h32_nk32768_d128", B=16, H=32, Nq=1, Nk=32768, d=128, dtype="bf16", kv_dtype="e4m3",
            causal=False, seed=8000, num_splits=64,
            description="1-token decode against an FP8 (E4M3) KV cache with a scale per (batch, head), "
                        "64-way split-KV + combine"),
        Workload(
            "masked_docs_b4h16_n8192_d128", B=4, H=16, Nq=8192, Nk=8192, d=128, dtype="bf16", causal=False,
            seed=10000, mask_rule=("documents", 10001, 256, 3072),
            description="8192 tokens packed from documents of 256 to 3072 tokens (seeded lengths), each token "
                        "attending causally within its own document; one element mask for every batch and head"),
        Workload(
            "prefill_fp8_b8h16_n8192_d128_causal", B=8, H=16, Nq=8192, Nk=8192, d=128, dtype="bf16",
            kv_dtype="e4m3", q_dtype="e4m3", causal=True, seed=9000, k_rule=("scale_all", 2.0),
            description="the headline causal prefill with Q, K and V as FP8 (E4M3) codes, a scale per "
                        "(batch, head) and tensor; O in bf16"),
    ]
}

PREFILL_HEADLINE = "prefill_b8h16_n8192_d128_causal"
DECODE_HEADLINE = "decode_b16h32_nk32768_d128"


def get(name: str) -> Workload:
    return WORKLOADS[name]
