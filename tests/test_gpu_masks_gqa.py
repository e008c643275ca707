"""Parity of the extended entry points (fa_fwd_ex, fa_decode_split_ex through the C ABI) with the
float64 reference: grouped K/V heads and both causal alignments (top-left for any Nq, Nk;
bottom-right for a query chunk appended to a KV cache).

Small shapes are compared element by element over the whole output (ragged tiles, Nq < Nk and
Nq > Nk, one query, several group sizes).  In the forward, grouped heads must give bit-for-bit
what the same kernel gives on K/V with each head repeated, and the extended entry points with
H_kv = H must give bit-for-bit what fa_fwd / fa_decode_split give.  The grouped decode split runs
both products on the matrix core (the ungrouped one on the VALU), so grouped against repeated
heads is held to the reference's tolerance instead.  The full-size chunked-prefill and grouped
decode workloads, and shapes with more query blocks than compute units, are compared on every
head in tests/test_gpu_workloads_all_heads.py."""

import numpy as np
import pytest
import torch

import exact_attention_126_amd as fa
import oracle
from synth import inputs as si
from synth.workloads import Workload
from tests.gpu_util import assert_parity, device_inputs, from_device, metrics

pytestmark = pytest.mark.gpu

MASK_OF = {None: fa.FA_MASK_NONE, "top_left": fa.FA_MASK_CAUSAL, "bottom_right": fa.FA_MASK_CAUSAL_BOTTOM_RIGHT}


def _fw(name, B, H, Hkv, Nq, Nk, d, dtype, align, k_rule=("none",), seed=21):
    return Workload(name, B=B, H=H, H_kv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype=dtype, causal=align is not None, seed=seed,
                    k_rule=k_rule, causal_align=align or "top_left")


FWD_SMALL = [
    _fw("br_nq300_nk1000_g4", 1, 4, 1, 300, 1000, 128, "bf16", "bottom_right"),
    _fw("tl_n513_g4_b2", 2, 8, 2, 513, 513, 128, "bf16", "top_left", ("scale_all", 2.0)),
    _fw("tl_nq700_nk300", 1, 4, 4, 700, 300, 128, "bf16", "top_left"),
    _fw("tl_nq200_nk900_g2", 1, 2, 1, 200, 900, 128, "bf16", "top_left"),
    _fw("br_nq1_nk777", 1, 8, 8, 1, 777, 128, "bf16", "bottom_right"),
    _fw("br_nq256_nk4096_g2", 1, 4, 2, 256, 4096, 128, "bf16", "bottom_right", ("scale_rows_every", 64, 8.0)),
    _fw("none_nq333_nk555_g8_b2", 2, 8, 1, 333, 555, 128, "bf16", None),
    _fw("br_nq129_nk700_d64_g2", 1, 6, 3, 129, 700, 64, "bf16", "bottom_right"),
    _fw("tl_nq1000_nk64_d64", 1, 2, 1, 1000, 64, 64, "bf16", "top_left"),
    _fw("br_nq64_nk64_d64", 1, 2, 2, 64, 64, 64, "bf16", "bottom_right"),
    _fw("f32_br_nq100_nk300", 1, 2, 1, 100, 300, 128, "f32", "bottom_right"),
    _fw("f32_tl_nq150_nk90", 1, 2, 2, 150, 90, 64, "f32", "top_left"),
    _fw("f32_none_n77_g2", 1, 4, 2, 77, 77, 64, "f32", None),
]


def _fwd_ex(w, dev):
    align = w.causal_align if w.causal else None
    print(f"  [fa_fwd_ex] {w.name}: B={w.B} H={w.H} H_kv={w.kv_heads} Nq={w.Nq} Nk={w.Nk} d={w.d} {w.dtype} "
          f"mask={align} seed={w.seed}", flush=True)
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    fa.fa_fwd_ex(dev["q"], dev["k"], dev["v"], o, lse, MASK_OF[align], w.scale)
    torch.cuda.synchronize()
    return o, lse


def _ref(w, host):
    return oracle.attention(si.as_f32(w, host["q"]), si.as_f32(w, host["k"]), si.as_f32(w, host["v"]), w.scale,
                            w.causal, diag=w.diag)


@pytest.mark.parametrize("w", FWD_SMALL, ids=lambda w: w.name)
def test_fwd_ex_small_full_compare(w):
    host, dev = device_inputs(w)
    o, lse = _fwd_ex(w, dev)
    o_ref, l_ref = _ref(w, host)
    assert_parity(w.dtype, metrics(from_device(o), from_device(lse), o_ref, l_ref), w.name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_grouped_heads_equal_repeated_heads_bitwise(dtype):
    w = _fw("gqa_vs_repeat", 2, 8, 2, 300, 700, 128, dtype, "bottom_right")
    _, dev = device_inputs(w)
    o, lse = _fwd_ex(w, dev)
    rep = {x: dev[x].repeat_interleave(w.H // w.kv_heads, dim=1).contiguous() for x in "kv"}
    o2 = torch.empty_like(o)
    l2 = torch.empty_like(lse)
    print("  [fa_fwd_ex] same inputs, K/V heads repeated", flush=True)
    fa.fa_fwd_ex(dev["q"], rep["k"], rep["v"], o2, l2, fa.FA_MASK_CAUSAL_BOTTOM_RIGHT, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16) if dtype == "bf16" else o, o2.view(torch.int16) if dtype == "bf16" else o2)
    assert torch.equal(lse, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_ex_with_all_heads_equals_fa_fwd_bitwise(causal):
    w = _fw("ex_vs_fwd", 1, 4, 4, 513, 513, 128, "bf16", "top_left" if causal else None)
    _, dev = device_inputs(w)
    o, lse = _fwd_ex(w, dev)
    print(f"  [fa_fwd] same inputs, causal={causal}", flush=True)
    o2, l2 = fa.attention(dev["q"], dev["k"], dev["v"], causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


def test_bottom_right_equals_top_left_when_square_bitwise():
    w = _fw("br_vs_tl", 1, 2, 1, 300, 300, 64, "bf16", "bottom_right")
    _, dev = device_inputs(w)
    o, lse = _fwd_ex(w, dev)
    o2 = torch.empty_like(o)
    l2 = torch.empty_like(lse)
    fa.fa_fwd_ex(dev["q"], dev["k"], dev["v"], o2, l2, fa.FA_MASK_CAUSAL, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


# ------------------------------------------------------------------------------- decode
def _dw(name, B, H, Hkv, Nk, d, dtype, S, seed=31):
    return Workload(name, B=B, H=H, H_kv=Hkv, Nq=1, Nk=Nk, d=d, dtype=dtype, causal=False, seed=seed, num_splits=S)


DEC_SMALL = [
    _dw("g4_nk5000_s16", 2, 8, 2, 5000, 128, "bf16", 16),
    _dw("g8_nk100_s64_empty", 1, 8, 1, 100, 128, "bf16", 64),
    _dw("g2_nk777_s5_d64", 1, 6, 3, 777, 64, "bf16", 5),
    _dw("g4_nk50_s3_d64", 1, 4, 1, 50, 64, "bf16", 3),
    _dw("g2_nk1_s1", 1, 2, 1, 1, 128, "bf16", 1),
    _dw("g4_nk2049_s4_kv3", 2, 12, 3, 2049, 128, "bf16", 4),
    _dw("f32_g4_nk333_s7", 1, 4, 1, 333, 64, "f32", 7),
]


def _decode_ex(w, dev):
    print(f"  [fa_decode_split_ex] {w.name}: B={w.B} H={w.H} H_kv={w.kv_heads} Nk={w.Nk} d={w.d} {w.dtype} "
          f"splits={w.num_splits}", flush=True)
    o, lse = fa.decode(dev["q"], dev["k"], dev["v"], w.num_splits, w.scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("w", DEC_SMALL, ids=lambda w: w.name)
def test_decode_ex_small(w):
    host, dev = device_inputs(w)
    o, lse = _decode_ex(w, dev)
    o_ref, l_ref = _ref(w, host)
    assert_parity(w.dtype, metrics(from_device(o), from_device(lse), o_ref, l_ref), w.name)


@pytest.mark.parametrize("d", [128, 64])
def test_decode_grouped_matches_repeated_heads(d):
    """The grouped split (both products on the matrix core) and the ungrouped split on the same
    inputs with the K/V heads repeated: each within the decode tolerance of the float64 reference,
    and the two within twice that of each other."""
    w = _dw(f"dec_gqa_vs_repeat_d{d}", 2, 8, 2, 3000, d, "bf16", 16)
    host, dev = device_inputs(w)
    o, lse = _decode_ex(w, dev)
    rep = {x: dev[x].repeat_interleave(w.H // w.kv_heads, dim=1).contiguous() for x in "kv"}
    print("  [fa_decode_split] same inputs, K/V heads repeated", flush=True)
    o2, l2 = fa.decode(dev["q"], rep["k"], rep["v"], w.num_splits, w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = _ref(w, host)
    assert_parity("bf16", metrics(from_device(o), from_device(lse), o_ref, l_ref), w.name + " grouped")
    assert_parity("bf16", metrics(from_device(o2), from_device(l2), o_ref, l_ref), w.name + " repeated")
    og, orp = from_device(o).astype(np.float64), from_device(o2).astype(np.float64)
    assert np.abs(og - orp).max() <= 4e-2
    assert np.abs(from_device(lse) - from_device(l2)).max() <= 2e-3
