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
