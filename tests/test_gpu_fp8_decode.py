"""Parity of decode over an FP8 KV cache (fa_decode_split_fp8kv + fa_decode_combine through the C
ABI) with the float64 reference that decodes the same E4M3 codes from their definition
(oracle.attention_head_fp8kv).

The reference sees exactly the values the kernel sees (codes times per-head scale), so the bf16
tolerances of the other decode tests apply unchanged: the only differences are fp32 accumulation
order, folding the K scale into q, and the bf16 rounding of O.  Small shapes are compared over
every head (ragged splits, empty splits, group sizes 1, 3, 4, 8, d = 64 and 128); the full-size
workload runs as the benchmark times it and is compared on sampled heads.  Grouped heads must give
bit for bit what the same kernel gives on K/V (and scales) repeated per query head, and a NaN code
must poison exactly the query heads that read its K/V head."""
import numpy as np
import pytest
import torch

import exact_attention_126_amd as fa
import oracle
import synth
from synth import inputs as si
from synth.workloads import Workload
from tests.gpu_util import assert_parity, from_device, metrics, to_device

pytestmark = pytest.mark.gpu


def _w(name, B, H, Hkv, Nk, d, S, seed=81, k_rule=("none",)):
    return Workload(name, B=B, H=H, H_kv=Hkv, Nq=1, Nk=Nk, d=d, dtype="bf16", causal=False, seed=seed, num_splits=S,
                    kv_dtype="e4m3", k_rule=k_rule)


SMALL = [
    _w("g4_nk5000_s16", 2, 8, 2, 5000, 128, 16),
    _w("g8_nk100_s64_empty", 1, 8, 1, 100, 128, 64),
    _w("g3_nk777_s5_d64", 1, 6, 2, 777, 64, 5),
    _w("g1_nk333_s7", 2, 4, 4, 333, 128, 7, k_rule=("scale_all", 2.0)),
    _w("g2_nk4097_s32_d64", 1, 4, 2, 4097, 64, 32),
    _w("g4_nk1_s1", 1, 4, 1, 1, 128, 1),
]


def _inputs(w):
    q = si.make_tensor(w, "q")
    kc, ks = si.make_kv_fp8(w, "k")
    vc, vs = si.make_kv_fp8(w, "v")
    host = {"q": q, "k": kc, "v": vc, "ks": ks, "vs": vs}
    dev = {"q": to_device(w, q), "k": torch.from_numpy(kc).cuda(), "v": torch.from_numpy(vc).cuda(),
           "ks": torch.from_numpy(ks).cuda(), "vs": torch.from_numpy(vs).cuda()}
    return host, dev


def _run(w, dev):
    print(f"  [fa_decode_split_fp8kv] {w.name}: B={w.B} H={w.H} H_kv={w.kv_heads} Nk={w.Nk} d={w.d} "
          f"splits={w.num_splits} seed={w.seed}", flush=True)
    o, lse = fa.decode_fp8kv(dev["q"], dev["k"], dev["v"], dev["ks"], dev["vs"], w.num_splits, w.scale)
    torch.cuda.synchronize()
    return o, lse


def _ref_head(w, host, b, h):
    grp = w.H // w.kv_heads
    hk = h // grp
    return oracle.attention_head_fp8kv(si.as_f32(w, host["q"][b, h]), host["k"][b, hk], host["v"][b, hk],
                                       host["ks"][b, hk], host["vs"][b, hk], w.scale)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fp8kv_decode_small_every_head(w):
    host, dev = _inputs(w)
    o, lse = _run(w, dev)
    o_h, l_h = from_device(o), from_device(lse)
    refs = [_ref_head(w, host, b, h) for b in range(w.B) for h in range(w.H)]
    r_o = np.stack([r[0] for r in refs]).reshape(o_h.shape)
    r_l = np.stack([r[1] for r in refs]).reshape(l_h.shape)
    assert_parity("bf16", metrics(o_h, l_h, r_o, r_l), w.name)


def test_fp8kv_grouped_equals_repeated_bitwise():
    w = _w("fp8_gqa_vs_repeat", 2, 8, 2, 3000, 128, 16)
    _, dev = _inputs(w)
    o, lse = _run(w, dev)
    rep = {x: dev[x].repeat_interleave(w.H // w.kv_heads, dim=1).contiguous() for x in ("k", "v", "ks", "vs")}
    print("  [fa_decode_split_fp8kv] same inputs, K/V heads and scales repeated", flush=True)
    o2, l2 = fa.decode_fp8kv(dev["q"], rep["k"], rep["v"], rep["ks"], rep["vs"], w.num_splits, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


def test_fp8kv_nan_code_poisons_its_group_only():
    """E4M3 has no infinity; S.1111.111 is NaN.  One NaN code in K/V head (0, 1) makes the query
    heads of that group NaN and leaves every other head bit for bit as it was."""
    w = _w("fp8_nan", 2, 8, 2, 1000, 128, 8)
    _, dev = _inputs(w)
    o, lse = _run(w, dev)
    k2 = dev["k"].clone()
    k2[0, 1, 517, 9] = 0x7F
    print("  [fa_decode_split_fp8kv] one K code set to NaN", flush=True)
    o2, l2 = fa.decode_fp8kv(dev["q"], k2, dev["v"], dev["ks"], dev["vs"], w.num_splits, w.scale)
    torch.cuda.synchronize()
    grp = w.H // w.kv_heads
    bad = torch.zeros(w.B, w.H, dtype=torch.bool)
    bad[0, grp:2 * grp] = True
    of, o2f = o.float().cpu(), o2.float().cpu()
    assert torch.isnan(o2f[bad]).all() and torch.isnan(l2.cpu()[bad]).all()
    assert torch.equal(o.view(torch.int16).cpu()[~bad], o2.view(torch.int16).cpu()[~bad])
    assert torch.equal(lse.cpu()[~bad], l2.cpu()[~bad]) and not torch.isnan(of).any()


def test_fp8kv_decode_workload_sampled_heads():
    """B16 H32 Nk32768 d128 over an E4M3 cache, 64 splits, as the benchmark times it: 24 heads."""
    w = synth.get("decode_fp8kv_b16h32_nk32768_d128")
    host, dev = _inputs(w)
    o, lse = _run(w, dev)
    o_h, l_h = from_device(o), from_device(lse)
    g = np.random.default_rng(8)
    heads = [(0, 0), (15, 31), (3, 4), (3, 7)] + [tuple(x) for x in zip(g.integers(0, 16, 20), g.integers(0, 32, 20))]
    refs = [_ref_head(w, host, b, h) for b, h in heads]
    got_o = np.stack([o_h[b, h] for b, h in heads])
    got_l = np.stack([l_h[b, h] for b, h in heads])
    assert_parity("bf16", metrics(got_o, got_l, np.stack([r[0] for r in refs]), np.stack([r[1] for r in refs])),
                  w.name)
