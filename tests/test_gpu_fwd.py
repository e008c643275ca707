"""Parity of the fused forward (fa_fwd through the C ABI) with the float64 reference.

Small shapes are compared element by element over the whole output: they span several
64-key tiles and 128-row query blocks with ragged tails.  The full-size workloads run in the
same launch configuration the benchmark times and are compared on sampled rows of sampled
heads, which the reference computes one by one."""
import math

import numpy as np
import pytest
import torch

import exact_attention_126_amd as fa
import oracle
import synth
from synth import inputs as si
from synth.workloads import Workload
from tests.gpu_util import assert_parity, device_inputs, from_device, metrics, sample_rows

pytestmark = pytest.mark.gpu


def _small(name, B, H, Nq, Nk, d, dtype, causal, k_rule=("none",), seed=7):
    return Workload(name, B=B, H=H, Nq=Nq, Nk=Nk, d=d, dtype=dtype, causal=causal, seed=seed, k_rule=k_rule)


SMALL = [
    _small("one_by_one", 1, 1, 1, 1, 64, "bf16", False),
    _small("nq1_nk7", 1, 1, 1, 7, 128, "bf16", False),
    _small("nq5_nk3_h2", 1, 2, 5, 3, 64, "bf16", False),
    _small("n64_causal", 1, 1, 64, 64, 128, "bf16", True),
    _small("n65_causal", 1, 1, 65, 65, 64, "bf16", True),
    _small("n127_causal_b2h3", 2, 3, 127, 127, 128, "bf16", True, ("scale_all", 2.0)),
    _small("nq129_nk200", 1, 2, 129, 200, 128, "bf16", False),
    _small("n300_causal_rows8", 2, 2, 300, 300, 128, "bf16", True, ("scale_rows_every", 64, 8.0)),
    _small("nq257_nk1000", 1, 1, 257, 1000, 64, "bf16", False, ("scale_all", 2.0)),
    _small("nq1000_nk37", 1, 1, 1000, 37, 128, "bf16", False),
    _small("n513_causal_d64", 1, 2, 513, 513, 64, "bf16", True),
    _small("f32_n1", 1, 1, 1, 1, 64, "f32", False),
    _small("f32_n77_causal", 1, 2, 77, 77, 128, "f32", True),
    _small("f32_nq130_nk33", 2, 1, 130, 33, 64, "f32", False),
    _small("f32_n300_causal", 1, 1, 300, 300, 64, "f32", True, ("scale_rows_every", 64, 8.0)),
    _small("f32_nq40_nk700", 1, 1, 40, 700, 128, "f32", False, ("scale_all", 2.0)),
]


def _run(w, dev):
    print(f"  [fa_fwd] {w.name}: B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d} {w.dtype} causal={w.causal} "
          f"seed={w.seed}", flush=True)
    o, lse = fa.attention(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fwd_small_full_compare(w):
    host, dev = device_inputs(w)
    o, lse = _run(w, dev)
    o_ref, l_ref = oracle.attention(si.as_f32(w, host["q"]), si.as_f32(w, host["k"]), si.as_f32(w, host["v"]),
                                    w.scale, w.causal)
    assert_parity(w.dtype, metrics(from_device(o), from_device(lse), o_ref, l_ref), w.name)


def test_tiny_f32_workload_full():
    w = synth.get("tiny_f32_n128_d64")
    host, dev = device_inputs(w)
    o, lse = _run(w, dev)
    o_ref, l_ref = oracle.attention(host["q"], host["k"], host["v"], w.scale, w.causal)
    assert_parity("f32", metrics(from_device(o), from_device(lse), o_ref, l_ref), w.name)


def test_short_batch_workload_heads():
    """B4 H16 N2048 d64: every row of six heads spread over the batch and head indices."""
    w = synth.get("batch_b4h16_n2048_d64")
    host, dev = device_inputs(w)
    o, lse = _run(w, dev)
    o_h, l_h = from_device(o), from_device(lse)
    for b, h in [(0, 0), (0, 15), (1, 7), (2, 3), (3, 0), (3, 15)]:
        o_ref, l_ref = oracle.attention_head(si.as_f32(w, host["q"][b, h]), si.as_f32(w, host["k"][b, h]),
                                             si.as_f32(w, host["v"][b, h]), w.scale, w.causal)
        assert_parity("bf16", metrics(o_h[b, h], l_h[b, h], o_ref, l_ref), f"{w.name} b={b} h={h}")


def _sampled_causal_workload(name, heads, nrows):
    w = synth.get(name)
    host, dev = device_inputs(w)
    o, lse = _run(w, dev)
    o_h, l_h = from_device(o), from_device(lse)
    del dev, o, lse
    for i, (b, h) in enumerate(heads):
        rows = sample_rows(w.Nq, nrows, seed=100 + i)
        o_ref, l_ref = oracle.attention_head(si.as_f32(w, host["q"][b, h]), si.as_f32(w, host["k"][b, h]),
                                             si.as_f32(w, host["v"][b, h]), w.scale, w.causal, rows=rows)
        assert_parity("bf16", metrics(o_h[b, h][rows], l_h[b, h][rows], o_ref, l_ref),
                      f"{w.name} b={b} h={h} rows={len(rows)}")


def test_headline_prefill_sampled():
    """B8 H16 N8192 d128 causal, K x2: sampled rows of four heads."""
    _sampled_causal_workload("prefill_b8h16_n8192_d128_causal", [(0, 0), (3, 9), (5, 2), (7, 15)], 384)


def test_long_context_sampled():
    """B1 H32 N16384 d128 causal, every 64th key row x8: sampled rows of three heads."""
    _sampled_causal_workload("long_b1h32_n16384_d128_causal", [(0, 0), (0, 17), (0, 31)], 384)


def test_lse_matches_log_of_row_sum_identity():
    """LSE is in natural-log units: with Q = 0 it is ln(#allowed keys) exactly up to rounding."""
    w = _small("zero_q", 1, 2, 200, 200, 128, "bf16", True)
    host, dev = device_inputs(w)
    dev["q"].zero_()
    o, lse = _run(w, dev)
    expect = np.log(np.arange(1, 201, dtype=np.float64))
    assert np.abs(from_device(lse)[0, 0] - expect).max() < 1e-5
