"""Parity of the forward with FP8 inputs (fa_fwd_fp8 through the C ABI) with the float64
reference on the same E4M3 codes and scales (oracle.attention_head_fp8).

Tolerance, derived from the arithmetic of the kernel (the reference sees the decoded values
exactly, so only the kernel's own roundings count).  For query row i, with p_j = exp(s_ij - max_j
s_ij) and l = sum_j p_j from the reference:
  * scores: the FP8 matrix core accumulates the 64-term code products in fp32 with an error we
    bound by eps_mma = 2^-11 of sum_d |q_d k_d| (measured on this hardware: at most 2^-12.9 over
    random codes of every magnitude), so each p_j carries a relative error of at most
    eta_i = exp(scale * eps_mma * max_j sum_d |q_id k_jd|) - 1;
  * P is rounded to E4M3 with round-to-nearest-even: relative error <= 2^-4 where it is normal,
    absolute <= 2^-10 in the kernel's units, which are at least 2^4 times the units of p_j (the
    kernel keeps its values between 2^-10 and 2^8 of its running max), i.e. <= 2^-14 * l-units;
  * the second product accumulates with the same eps_mma; O is rounded to bf16 (<= 2^-9).
So every element obeys
  |O_gpu - O_ref|_ic <= (2^-4 + 2 eta_i + 2 eps_mma) sum_j w_j |v_jc| + 2^-14 sum_j |v_jc| / l
                        + 2^-8 |O_ref,ic| + 1e-6,            w_j = p_j / l,
and the LSE (from the unrounded P) obeys |LSE_gpu - LSE_ref|_i <= log(1 + eta_i) + 1e-5 (1 + |LSE|).
Beside the element-wise bound, the relative L2 error of O is held to 4e-2: independent
round-to-nearest errors of a 3-bit mantissa have an RMS relative size of at most 2^-4 / sqrt(3),
about 3.6e-2, and the output error is their w-weighted average over V.
"""
import numpy as np
import pytest
import torch

import exact_attention_126_amd as fa
import oracle
import synth
from synth import inputs as si
from synth.workloads import Workload
from tests.gpu_util import from_device, sample_rows, to_device

pytestmark = pytest.mark.gpu

EPS_MMA = 2.0 ** -11
O_REL_L2 = 4e-2
MASK_OF = {None: fa.FA_MASK_NONE, "top_left": fa.FA_MASK_CAUSAL, "bottom_right": fa.FA_MASK_CAUSAL_BOTTOM_RIGHT}


def _w(name, B, H, Hkv, Nq, Nk, d, align, k_rule=("none",), seed=91):
    return Workload(name, B=B, H=H, H_kv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype="bf16", causal=align is not None, seed=seed,
                    k_rule=k_rule, causal_align=align or "top_left", kv_dtype="e4m3", q_dtype="e4m3")


SMALL = [
    _w("n64_d128", 1, 2, 2, 64, 64, 128, None),
    _w("n300_causal_k2", 1, 2, 2, 300, 300, 128, "top_left", ("scale_all", 2.0)),
    _w("nq257_nk513_br_g2", 2, 4, 2, 257, 513, 128, "bottom_right"),
    _w("nq100_nk700_d64", 1, 2, 1, 100, 700, 64, None),
    _w("n129_causal_d64_g4", 1, 4, 1, 129, 129, 64, "top_left"),
    _w("nq1_nk333_br", 1, 2, 2, 1, 333, 128, "bottom_right"),
    _w("nq300_nk100_tl", 1, 2, 2, 300, 100, 128, "top_left"),
    _w("n520_causal_rows8", 1, 2, 2, 520, 520, 128, "top_left", ("scale_rows_every", 64, 8.0)),
    _w("n1000_none_k2_b2", 2, 2, 1, 1000, 1000, 128, None, ("scale_all", 2.0)),
]


def _inputs(w):
    host, dev = {}, {}
    for x in "qkv":
        codes, scales = si.make_kv_fp8(w, x)
        host[x], host[x + "s"] = codes, scales
        dev[x], dev[x + "s"] = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    return host, dev


def _run(w, dev):
    align = w.causal_align if w.causal else None
    print(f"  [fa_fwd_fp8] {w.name}: B={w.B} H={w.H} H_kv={w.kv_heads} Nq={w.Nq} Nk={w.Nk} d={w.d} mask={align} "
          f"seed={w.seed}", flush=True)
    o, lse = fa.attention_fp8(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], dev["vs"], MASK_OF[align], w.scale)
    torch.cuda.synchronize()
    return o, lse


def _head_check(w, host, b, h, o_gpu, lse_gpu, rows=None):
    """Reference and bounds for one head (rows: the query rows o_gpu / lse_gpu hold, or all)."""
    grp = w.H // w.kv_heads
    hk = h // grp
    rows = np.arange(w.Nq) if rows is None else np.asarray(rows)
    o_ref, l_ref = oracle.attention_head_fp8(host["q"][b, h], host["k"][b, hk], host["v"][b, hk], host["qs"][b, h],
                                             host["ks"][b, hk], host["vs"][b, hk], w.scale, w.causal, rows=rows,
                                             diag=w.diag)
    # the quantities the bound needs, from the decoded values (float64)
    q = oracle.e4m3_decode(host["q"][b, h][rows]) * float(host["qs"][b, h])
    k = oracle.e4m3_decode(host["k"][b, hk]) * float(host["ks"][b, hk])
    v = oracle.e4m3_decode(host["v"][b, hk]) * float(host["vs"][b, hk])
    s = w.scale * (q @ k.T)
    if w.causal:
        s = np.where(np.arange(w.Nk)[None, :] > rows[:, None] + w.diag, -np.inf, s)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    l = p.sum(axis=1, keepdims=True)
    vis = np.isfinite(s).astype(np.float64)
    eta = np.expm1(w.scale * EPS_MMA * (np.abs(q) @ np.abs(k).T * vis).max(axis=1, keepdims=True))
    av = np.abs(v)
    bound = ((2.0 ** -4 + 2 * eta + 2 * EPS_MMA) * ((p / l) @ av) + 2.0 ** -14 * (vis @ av) / l
             + 2.0 ** -8 * np.abs(o_ref) + 1e-6)
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    lse_bound = np.log1p(eta[:, 0]) + 1e-5 * (1 + np.abs(l_ref))
    lse_err = np.abs(lse_gpu.astype(np.float64) - l_ref)
    return o_ref, l_ref, float((err / bound).max()), float((lse_err / lse_bound).max())


def _check(w, host, o, lse, heads, rows=None):
    o_h, l_h = from_device(o), from_device(lse)
    got, ref, worst, worst_l = [], [], 0.0, 0.0
    for b, h in heads:
        og = o_h[b, h] if rows is None else o_h[b, h][rows]
        lg = l_h[b, h] if rows is None else l_h[b, h][rows]
        o_ref, _, r_o, r_l = _head_check(w, host, b, h, og, lg, rows)
        got.append(og)
        ref.append(o_ref)
        worst, worst_l = max(worst, r_o), max(worst_l, r_l)
    got, ref = np.stack(got).astype(np.float64), np.stack(ref)
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"    {w.name}: O rel-L2 {rel:.3e}, worst |err|/bound O {worst:.3f}, LSE {worst_l:.3f}", flush=True)
    assert np.isfinite(got).all()
    assert worst <= 1.0 and worst_l <= 1.0, (w.name, worst, worst_l)
    assert rel <= O_REL_L2, (w.name, rel)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fwd_fp8_small_every_head(w):
    host, dev = _inputs(w)
    o, lse = _run(w, dev)
    _check(w, host, o, lse, [(b, h) for b in range(w.B) for h in range(w.H)])


def test_fwd_fp8_grouped_equals_repeated_bitwise():
    w = _w("fp8_gqa_vs_repeat", 2, 8, 2, 300, 700, 128, "bottom_right")
    _, dev = _inputs(w)
    o, lse = _run(w, dev)
    rep = {x: dev[x].repeat_interleave(w.H // w.kv_heads, dim=1).contiguous() for x in ("k", "v", "ks", "vs")}
    print("  [fa_fwd_fp8] same inputs, K/V heads and scales repeated", flush=True)
    o2, l2 = fa.attention_fp8(dev["q"], rep["k"], rep["v"], dev["qs"], rep["ks"], rep["vs"],
                              fa.FA_MASK_CAUSAL_BOTTOM_RIGHT, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


def test_fwd_fp8_reproducible():
    w = _w("fp8_repro", 1, 4, 4, 600, 600, 128, "top_left")
    _, dev = _inputs(w)
    a = _run(w, dev)
    b = _run(w, dev)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_fwd_fp8_prefill_workload_sampled():
    """B8 H16 N8192 d128 causal with E4M3 Q, K, V, as the benchmark times it: sampled rows of
    three heads against the reference and the bound."""
    w = synth.get("prefill_fp8_b8h16_n8192_d128_causal")
    host, dev = _inputs(w)
    o, lse = _run(w, dev)
    rows = sample_rows(w.Nq, 192, seed=300)
    _check(w, host, o, lse, [(0, 0), (3, 9), (7, 15)], rows)
