"""Parity of the fused forward (fa_fwd through the C ABI) with the float64 reference.

Small shapes are compared element by element over the whole output: they span several
64-key tiles and 128-row query blocks with ragged tails.  The full-size workloads are compared
on every head in tests/test_gpu_workloads_all_heads.py."""
import numpy as np
import pytest
import torch

import exact_attention_126_amd as fa
import oracle
from synth import inputs as si
from synth.workloads import Workload
from tests.gpu_util import assert_parity, device_inputs, from_device, metrics

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


def test_lse_matches_log_of_row_sum_identity():
    """LSE is in natural-log units: with Q = 0 it is ln(#allowed keys) exactly up to rounding."""
    w = _small("zero_q", 1, 2, 200, 200, 128, "bf16", True)
    host, dev = device_inputs(w)
    dev["q"].zero_()
    o, lse = _run(w, dev)
    expect = np.log(np.arange(1, 201, dtype=np.float64))
    assert np.abs(from_device(lse)[0, 0] - expect).max() < 1e-5
