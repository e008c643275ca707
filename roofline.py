"""Algorithmic work, byte counts and MI355X peaks used to place the kernels on a roofline
(measurement only: the benchmark and the tests use it, the library does not).

Conventions:
  * attention FLOPs = 4 * B * H * Nq * Nk * d (two dense contractions, Q K^T and P V, at
    2 FLOP per multiply-add), halved for a causal mask: only the lower triangle is live
    (Day-21 page §6 table and §8 thought question 3).  The extra exp/rescale work of the
    online softmax (Day-21 page §7) is not counted.
  * minimum HBM bytes = read Q, K, V once and write O and the fp32 LSE once.
  * the standard, unfused data flow moves each N x N matrix through HBM: S written and
    read, P written and read (Day-21 page §3.1 and §8 exercise 1).
"""
from __future__ import annotations

# MI355X published peaks.
PEAK_BF16_MFMA_TFLOPS = 2516.6  # dense: 256 CU x 2.4 GHz x 4096 FLOP/clk/CU
PEAK_FP8_MFMA_TFLOPS = 5033.2   # dense: 256 CU x 2.4 GHz x 8192 FLOP/clk/CU
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
CUS = 256
CLOCK_GHZ = 2.4


def attention_flops(B, H, Nq, Nk, d, causal) -> float:
    f = 4.0 * B * H * Nq * Nk * d
    return f / 2 if causal else f


def min_hbm_bytes(B, H, Nq, Nk, d, elt_bytes) -> int:
    """Q, K, V read once; O and the fp32 LSE written once."""
    return B * H * (Nq * d * elt_bytes * 2 + 2 * Nk * d * elt_bytes + Nq * 4)


def decode_kv_bytes(B, H, Nk, d, elt_bytes) -> int:
    """The KV cache read once: the whole algorithmic traffic of one decode step, up to
    q, O and LSE (a few hundred KB)."""
    return 2 * B * H * Nk * d * elt_bytes


def decode_min_bytes(B, H, Nk, d, elt_bytes) -> int:
    return decode_kv_bytes(B, H, Nk, d, elt_bytes) + B * H * (2 * d * elt_bytes + 4)


def score_matrix_elements(N) -> int:
    return N * N


def standard_attention_hbm_bytes(B, H, N, d, elt_bytes) -> int:
    """Unfused data flow: S written, S read, P written, P read (4 N^2 crossings) plus
    Q, K, V read and O written."""
    return B * H * (4 * N * N + 4 * N * d) * elt_bytes


def qblock_kv_model_bytes(B, H, N, d, elt_bytes, block_q, causal) -> int:
    """HBM bytes if every query block re-reads the K/V it needs with no cache reuse between
    workgroups, plus Q and O once (the per-Q-block data-movement model)."""
    nblk = -(-N // block_q)
    kv_row = 2 * d * elt_bytes
    total_rows = 0
    for qb in range(nblk):
        total_rows += min(N, (qb + 1) * block_q) if causal else N
    return B * H * (total_rows * kv_row + 2 * N * d * elt_bytes)
