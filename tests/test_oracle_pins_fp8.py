"""Pins of the FP8 (OCP E4M3) decoding in the float64 reference (CPU only).

Every one of the 256 codes is checked against torch's float8_e4m3fn decoding (an independent
implementation of the same OCP format), the format's landmark values are checked by hand, and
the attention over an FP8 cache is checked to be the plain attention over the decoded values
times their scale (the part already pinned elsewhere)."""
import math

import numpy as np
import torch

import oracle


def test_all_codes_match_torch_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(both_nan, np.isnan(ref)) and np.array_equal(both_nan, np.isnan(got))
    assert np.array_equal(got[~both_nan], ref[~both_nan])


def test_landmark_values():
    v = oracle.e4m3_value
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0      # +0 and -0
    assert v(0x38) == 1.0 and v(0xB8) == -1.0                            # exponent field 7 = bias
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0                        # largest finite
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))                    # the only NaNs
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9              # subnormals m/8 * 2^-6
    assert v(0x08) == 2.0 ** -6                                           # smallest normal
    assert v(0x78) == 256.0 and v(0x77) == 240.0                          # 1.0 * 2^8, 1.875 * 2^7


def test_finite_codes_are_monotone_in_magnitude():
    mags = [oracle.e4m3_value(c) for c in range(0x7F)]                    # 0x00 .. 0x7E
    assert all(a < b for a, b in zip(mags, mags[1:]))


def test_fp8_cache_attention_is_attention_on_decoded_values():
    g = np.random.default_rng(3)
    q = g.standard_normal((5, 8))
    kc = g.integers(0, 0x7F, (11, 8), dtype=np.uint8) | (g.integers(0, 2, (11, 8), dtype=np.uint8) << 7)
    vc = g.integers(0, 0x7F, (11, 8), dtype=np.uint8)
    o, lse = oracle.attention_head_fp8kv(q, kc, vc, 0.01, 0.02, 0.35)
    k = np.array([[oracle.e4m3_value(c) for c in row] for row in kc]) * 0.01
    v = np.array([[oracle.e4m3_value(c) for c in row] for row in vc]) * 0.02
    o2, l2 = oracle.attention_head(q, k, v, 0.35)
    assert np.abs(o - o2).max() < 1e-15 and np.abs(lse - l2).max() < 1e-15


def _brute_force_head(q, k, v, scale, causal):
    """Textbook softmax attention with Python loops (tiny inputs)."""
    out, lses = [], []
    for i in range(len(q)):
        keys = [j for j in range(len(k)) if not causal or j <= i]
        s = [scale * sum(a * b for a, b in zip(q[i], k[j])) for j in keys]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = sum(e)
        out.append([sum(e[t] * v[j][c] for t, j in enumerate(keys)) / tot for c in range(len(v[0]))])
        lses.append(mx + math.log(tot))
    return np.array(out), np.array(lses)


def test_fp8_inputs_attention_against_brute_force_on_decoded_codes():
    """Q, K, V all codes: the reference equals a pure-Python softmax over e4m3_value(code) * scale
    (no shared code path beyond the code table, itself pinned above)."""
    g = np.random.default_rng(4)
    for causal in (False, True):
        qc, kc, vc = (g.integers(0, 0x7F, (6, 4), dtype=np.uint8) | (g.integers(0, 2, (6, 4), dtype=np.uint8) << 7)
                      for _ in range(3))
        o, lse = oracle.attention_head_fp8(qc, kc, vc, 0.03, 0.02, 0.5, 0.7, causal)
        dq = [[oracle.e4m3_value(int(c)) * 0.03 for c in row] for row in qc]
        dk = [[oracle.e4m3_value(int(c)) * 0.02 for c in row] for row in kc]
        dv = [[oracle.e4m3_value(int(c)) * 0.5 for c in row] for row in vc]
        o2, l2 = _brute_force_head(dq, dk, dv, 0.7, causal)
        assert np.abs(o - o2).max() < 1e-12 * max(1.0, np.abs(o2).max()) and np.abs(lse - l2).max() < 1e-12


def test_fp8_scales_enter_only_through_their_products():
    """S depends on scale * q_scale * k_scale and O is linear in v_scale: moving a factor between
    them changes nothing (checks that no scale is dropped or applied twice)."""
    g = np.random.default_rng(5)
    qc, kc, vc = (g.integers(0, 0x7E, (9, 8), dtype=np.uint8) for _ in range(3))
    o1, l1 = oracle.attention_head_fp8(qc, kc, vc, 0.5, 0.25, 3.0, 0.1, True)
    o2, l2 = oracle.attention_head_fp8(qc, kc, vc, 0.25, 0.125, 1.0, 0.4, True)
    assert np.abs(o1 - 3.0 * o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12
