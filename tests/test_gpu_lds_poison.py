"""The LDS-poisoned build (libfa_poison.so, compiled with FA_DEBUG_POISON_LDS=1) against the normal
library, bit for bit.

In the poisoned build the waves that refill a slot of an LDS tile ring (K/V in the bf16 and FP8
forwards, K/V in dQ, Q/dO and the row statistics in dK/dV) first overwrite their part of it with
NaN, after the barrier that retires the slot and before their tile loads.  With every barrier in
place no wave reads the NaN, since the tile loads overwrite it first, so the two libraries must
give identical bits on every output.  A wave that read a slot before its tile had landed, or
after the slot was handed back for the next tile, would read NaN and turn its rows non-finite.
The shapes span many key tiles, ragged tails, causal diagonals, grouped K/V heads and
workgroups that walk several query blocks, so that every ring slot is refilled many times.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_attention_126_amd as fa
from exact_attention_126_amd import build as fa_build
from synth import inputs as si
from synth import masks
from synth.workloads import Workload
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu

MASK_OF = {None: fa.FA_MASK_NONE, "top_left": fa.FA_MASK_CAUSAL, "bottom_right": fa.FA_MASK_CAUSAL_BOTTOM_RIGHT}


@pytest.fixture(scope="module")
def libs():
    normal = fa.lib()
    poisoned = fa.load_library(fa_build.POISON_LIB)
    return normal, poisoned


def _both(libs, monkeypatch, fn):
    """fn() under the normal library, then under the poisoned one; both results, synchronized."""
    out = []
    for L in libs:
        monkeypatch.setattr(fa, "_lib", L)
        out.append(fn())
        torch.cuda.synchronize()
    monkeypatch.setattr(fa, "_lib", libs[0])
    return out


def _same_bits(a: torch.Tensor, b: torch.Tensor, what: str, finite: bool = True):
    assert a.shape == b.shape and a.dtype == b.dtype, what
    if finite:
        assert bool(torch.isfinite(a.float()).all()), f"{what}: normal build gives non-finite values"
        assert bool(torch.isfinite(b.float()).all()), f"{what}: poisoned build gives non-finite values"
    ia = a.contiguous().view(torch.uint8)
    ib = b.contiguous().view(torch.uint8)
    diff = int((ia != ib).sum())
    assert diff == 0, f"{what}: {diff} bytes differ between the normal and the poisoned build"


def _w(name, B, H, Hkv, Nq, Nk, d, align, seed=171, **kw):
    return Workload(name, B=B, H=H, H_kv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype="bf16", causal=align is not None, seed=seed,
                    causal_align=align or "top_left", **kw)


def _dev(w, names="qkv"):
    return {x: to_device(w, si.make_tensor(w, x)) for x in names}


def _fwd_ex(w, dev):
    align = w.causal_align if w.causal else None
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    fa.fa_fwd_ex(dev["q"], dev["k"], dev["v"], o, lse, MASK_OF[align], w.scale)
    return o, lse


FWD = [
    _w("fwd_causal_b2h3_n1000_d128", 2, 3, 3, 1000, 1000, 128, "top_left"),
    _w("fwd_none_nq300_nk777_d64", 1, 4, 4, 300, 777, 64, None),
    # more (block, head) items than compute units: workgroups walk several query blocks
    _w("fwd_causal_b2h16_n2048_d128", 2, 16, 16, 2048, 2048, 128, "top_left"),
    _w("fwd_causal_b2h16_n2048_d64", 2, 16, 16, 2048, 2048, 64, "top_left"),
]


@pytest.mark.parametrize("w", FWD, ids=lambda w: w.name)
def test_fwd_poisoned_matches(libs, monkeypatch, w):
    print(f"  [fa_fwd] {w.name}: B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d} causal={w.causal}", flush=True)
    dev = _dev(w)

    def run():
        o = torch.empty_like(dev["q"])
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
        fa.fa_fwd(dev["q"], dev["k"], dev["v"], o, lse, w.causal, w.scale)
        return o, lse

    (o0, l0), (o1, l1) = _both(libs, monkeypatch, run)
    _same_bits(o0, o1, f"{w.name} O")
    _same_bits(l0, l1, f"{w.name} LSE")


FWD_EX = [
    _w("fwd_ex_br_g2_nq257_nk513_d128", 2, 4, 2, 257, 513, 128, "bottom_right"),
    _w("fwd_ex_tl_g4_nq700_nk300_d64", 1, 8, 2, 700, 300, 64, "top_left"),
]


@pytest.mark.parametrize("w", FWD_EX, ids=lambda w: w.name)
def test_fwd_ex_poisoned_matches(libs, monkeypatch, w):
    print(f"  [fa_fwd_ex] {w.name}: B={w.B} H={w.H} H_kv={w.kv_heads} Nq={w.Nq} Nk={w.Nk} d={w.d} "
          f"mask={w.causal_align}", flush=True)
    dev = _dev(w)
    (o0, l0), (o1, l1) = _both(libs, monkeypatch, lambda: _fwd_ex(w, dev))
    # top-left alignment with Nq > Nk leaves no row empty here; every output is finite
    _same_bits(o0, o1, f"{w.name} O")
    _same_bits(l0, l1, f"{w.name} LSE")


def test_fwd_masked_poisoned_matches(libs, monkeypatch):
    w = Workload("masked_docs_b2h8_n1500_d128", B=2, H=8, H_kv=4, Nq=1500, Nk=1500, d=128, dtype="bf16",
                 causal=False, seed=173, mask_rule=("documents", 7, 60, 700))
    allowed = masks.element_mask(w)
    print(f"  [fa_fwd_masked] {w.name}: visible={masks.visible_pairs(allowed)}", flush=True)
    dev = _dev(w)
    md = torch.from_numpy(masks.pack_bits(allowed).view(np.int64)).cuda()

    def run():
        o = torch.empty_like(dev["q"])
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
        ws = torch.empty(fa.fa_fwd_masked_workspace_bytes(w.Nq, w.Nk), dtype=torch.uint8, device="cuda")
        fa.fa_fwd_masked(dev["q"], dev["k"], dev["v"], o, lse, md, ws, w.scale)
        return o, lse

    (o0, l0), (o1, l1) = _both(libs, monkeypatch, run)
    _same_bits(o0, o1, f"{w.name} O")
    _same_bits(l0, l1, f"{w.name} LSE")


FP8 = [
    _w("fp8_causal_b2h4_n1000_d128", 2, 4, 4, 1000, 1000, 128, "top_left", kv_dtype="e4m3", q_dtype="e4m3"),
    _w("fp8_none_g2_nq300_nk900_d64", 1, 4, 2, 300, 900, 64, None, kv_dtype="e4m3", q_dtype="e4m3"),
]


@pytest.mark.parametrize("w", FP8, ids=lambda w: w.name)
def test_fwd_fp8_poisoned_matches(libs, monkeypatch, w):
    print(f"  [fa_fwd_fp8] {w.name}: B={w.B} H={w.H} H_kv={w.kv_heads} Nq={w.Nq} Nk={w.Nk} d={w.d}", flush=True)
    dev = {}
    for x in "qkv":
        codes, scales = si.make_kv_fp8(w, x)
        dev[x], dev[x + "s"] = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    align = w.causal_align if w.causal else None
    (o0, l0), (o1, l1) = _both(libs, monkeypatch, lambda: fa.attention_fp8(
        dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], dev["vs"], MASK_OF[align], w.scale))
    _same_bits(o0, o1, f"{w.name} O")
    _same_bits(l0, l1, f"{w.name} LSE")


BWD = [
    _w("bwd_causal_b1h4_n1000_d128", 1, 4, 4, 1000, 1000, 128, "top_left"),
    _w("bwd_none_g2_nq300_nk700_d64", 1, 4, 2, 300, 700, 64, None),
    _w("bwd_br_g2_nq257_nk513_d128", 2, 4, 2, 257, 513, 128, "bottom_right"),
    _w("bwd_causal_b1h8_n2048_d64", 1, 8, 8, 2048, 2048, 64, "top_left"),
]


@pytest.mark.parametrize("w", BWD, ids=lambda w: w.name)
def test_bwd_poisoned_matches(libs, monkeypatch, w):
    align = w.causal_align if w.causal else None
    print(f"  [fa_bwd] {w.name}: B={w.B} H={w.H} H_kv={w.kv_heads} Nq={w.Nq} Nk={w.Nk} d={w.d} mask={align}",
          flush=True)
    dev = _dev(w, ("q", "k", "v", "do"))
    o, lse = _fwd_ex(w, dev)  # one forward (normal build) feeds both backward runs
    torch.cuda.synchronize()
    (g0, g1) = _both(libs, monkeypatch, lambda: fa.attention_backward(
        dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale=w.scale, mask=MASK_OF[align]))
    for name, a, b in zip(("dQ", "dK", "dV"), g0, g1):
        _same_bits(a, b, f"{w.name} {name}")
