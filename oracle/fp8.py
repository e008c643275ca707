"""OCP FP8 E4M3 values and attention over FP8 inputs, in float64 (test infrastructure only).

The Day-21 page's FAQ Q5 names KV-cache quantisation among the decode-side techniques (reading
the cache from HBM is the bottleneck there).  The reading taken: K and V stored as OCP FP8 E4M3
codes, each (batch, K/V head) with one float32 scale, the value of a code being its E4M3 value
times the scale; attention is then the plain definition in attention.py on those values.  The
Day-21 page (close of §6) names FP8 as a FlashAttention-3 feature; for the prefill the same
reading applies to Q as well: Q, K and V all E4M3 codes with one scale per (batch, head).

E4M3 (OCP 8-bit floating point, "E4M3FN"): sign bit, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 is subnormal (m / 8 * 2^-6); there are no infinities, and S.1111.111 is
NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_head


def e4m3_value(code: int) -> float:
    """The E4M3 value of one 8-bit code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """Array of uint8 codes -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def attention_head_fp8kv(q, k_codes, v_codes, k_scale: float, v_scale: float, scale: float, causal: bool = False,
                         rows=None, diag: int = 0):
    """One head against an FP8 KV cache: q [Nq, d] values, k/v [Nk, d] E4M3 codes with their
    scales -> (O, LSE) in float64."""
    k = e4m3_decode(k_codes) * float(k_scale)
    v = e4m3_decode(v_codes) * float(v_scale)
    return attention_head(q, k, v, scale, causal, rows=rows, diag=diag)


def attention_head_fp8(q_codes, k_codes, v_codes, q_scale: float, k_scale: float, v_scale: float, scale: float,
                       causal: bool = False, rows=None, diag: int = 0):
    """One head with Q, K and V all E4M3 codes ([Nq, d], [Nk, d], [Nk, d]) and their scales ->
    (O, LSE) in float64: the plain definition on the decoded values."""
    q = e4m3_decode(q_codes) * float(q_scale)
    return attention_head_fp8kv(q, k_codes, v_codes, k_scale, v_scale, scale, causal, rows=rows, diag=diag)
