"""Parity of the backward pass (fa_bwd through the C ABI) with the float64 reference gradients.

The GPU forward (fa_fwd_ex) produces O and LSE, the GPU backward takes them with a seeded dO;
the reference differentiates the plain definition (oracle.attention_backward), independently of
O and LSE.  Small shapes are compared over whole tensors: ragged query and key tiles, Nq < Nk and
Nq > Nk, both causal alignments, grouped K/V heads, d = 64 and 128.  Beside parity: the result is
bit-reproducible, and two identities the chain rule forces hold on the GPU output itself (the dK
rows of a K/V head sum to zero; its dV rows sum to the dO rows of its query heads).

Tolerance (tests/bwd_bounds.py, derived from the backward's arithmetic: P and dS rounded to bf16
before the products that consume them, fp32 accumulation, outputs rounded to bf16, and the
forward's own O and LSE errors, which the test knows): every element of dQ, dK and dV within its
worst-case bound, and each tensor's relative L2 error within 1.5 times the error predicted from
the same roundings taken as independent (3-7e-3 on these inputs)."""
import numpy as np
import pytest
import torch

import exact_attention_126_amd as fa
import oracle
from synth import inputs as si
from synth.workloads import Workload
from tests import bwd_bounds
from tests.gpu_util import from_device, to_device

pytestmark = pytest.mark.gpu

MASK_OF = {None: fa.FA_MASK_NONE, "top_left": fa.FA_MASK_CAUSAL, "bottom_right": fa.FA_MASK_CAUSAL_BOTTOM_RIGHT}


def _w(name, B, H, Hkv, Nq, Nk, d, align, k_rule=("none",), seed=41):
    return Workload(name, B=B, H=H, H_kv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype="bf16", causal=align is not None, seed=seed,
                    k_rule=k_rule, causal_align=align or "top_left")


SMALL = [
    _w("n64_d128", 1, 2, 2, 64, 64, 128, None),
    _w("n300_causal_d128", 1, 2, 2, 300, 300, 128, "top_left", ("scale_all", 2.0)),
    _w("nq257_nk513_br_g2", 2, 4, 2, 257, 513, 128, "bottom_right"),
    _w("nq100_nk700_d64", 1, 2, 1, 100, 700, 64, None),
    _w("n129_causal_d64_g4", 1, 4, 1, 129, 129, 64, "top_left"),
    _w("nq1_nk333_br", 1, 2, 2, 1, 333, 128, "bottom_right"),
    _w("nq300_nk100_tl", 1, 2, 2, 300, 100, 128, "top_left"),
    _w("n520_causal_rows8", 1, 2, 2, 520, 520, 128, "top_left", ("scale_rows_every", 64, 8.0)),
]


def _inputs(w):
    host = {x: si.make_tensor(w, x) for x in ("q", "k", "v", "do")}
    return host, {x: to_device(w, host[x]) for x in host}


def _run(w, dev, with_forward=False):
    align = w.causal_align if w.causal else None
    print(f"  [fa_fwd_ex + fa_bwd] {w.name}: B={w.B} H={w.H} H_kv={w.kv_heads} Nq={w.Nq} Nk={w.Nk} d={w.d} "
          f"mask={align} seed={w.seed}", flush=True)
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    fa.fa_fwd_ex(dev["q"], dev["k"], dev["v"], o, lse, MASK_OF[align], w.scale)
    dq, dk, dv = fa.attention_backward(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale=w.scale,
                                       mask=MASK_OF[align])
    torch.cuda.synchronize()
    if with_forward:
        return (dq, dk, dv), (o, lse)
    return dq, dk, dv


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_bwd_small_full_compare(w):
    host, dev = _inputs(w)
    (dq, dk, dv), (o, lse) = _run(w, dev, with_forward=True)
    f = {x: si.as_f32(w, host[x]) for x in host}
    res = bwd_bounds.reference_and_bounds(f["q"], f["k"], f["v"], f["do"], from_device(o), from_device(lse), w.scale,
                                          w.causal, w.diag)
    # the bound's reference is the definition; it must agree with the oracle's gradients
    rq, rk, rv = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], w.scale, w.causal, diag=w.diag)
    for x, r in (("dq", rq), ("dk", rk), ("dv", rv)):
        assert np.abs(res[x][0] - r).max() <= 1e-9 * max(1.0, np.abs(r).max())
    bwd_bounds.check({"dq": from_device(dq), "dk": from_device(dk), "dv": from_device(dv)}, res, w.name)


def test_bwd_bitwise_reproducible():
    w = _w("repro", 1, 4, 2, 600, 600, 128, "top_left")
    _, dev = _inputs(w)
    a = _run(w, dev)
    b = _run(w, dev)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_identities_on_gpu_output():
    """Per K/V head: sum over keys of dK is ~0 and sum over keys of dV equals the sum of dO rows
    of its query heads (every row's P sums to one)."""
    w = _w("identities", 1, 4, 2, 512, 768, 128, "bottom_right")
    host, dev = _inputs(w)
    dq, dk, dv = _run(w, dev)
    dk_h, dv_h = from_device(dk).astype(np.float64), from_device(dv).astype(np.float64)
    do = si.as_f32(w, host["do"]).astype(np.float64)
    grp = w.H // w.kv_heads
    for hk in range(w.kv_heads):
        sdk = dk_h[0, hk].sum(axis=0)
        assert np.abs(sdk).max() <= 2e-2 * np.abs(dk_h[0, hk]).sum(axis=0).max() + 1e-3, ("sum dK", hk)
        want = do[0, hk * grp:(hk + 1) * grp].sum(axis=(0, 1))
        got = dv_h[0, hk].sum(axis=0)
        assert np.abs(got - want).max() <= 1e-2 * np.abs(want).max() + 0.5, ("sum dV", hk, np.abs(got - want).max())


def test_bwd_prefill_one_kv_group():
    """B2 H8 H_kv2 N4096 d128 causal (grouped heads): the four query heads of one K/V head, whole
    heads, against the reference and the bounds (dQ of each query head, dK and dV of the K/V head)."""
    w = _w("bwd_b2h8kv2_n4096_d128_causal", 2, 8, 2, 4096, 4096, 128, "top_left", ("scale_all", 2.0), seed=43)
    host, dev = _inputs(w)
    (dq, dk, dv), (o, lse) = _run(w, dev, with_forward=True)
    b, hk = 1, 1
    grp = w.H // w.kv_heads
    hs = slice(hk * grp, (hk + 1) * grp)
    got = {"dq": from_device(dq)[b:b + 1, hs], "dk": from_device(dk)[b:b + 1, hk:hk + 1],
           "dv": from_device(dv)[b:b + 1, hk:hk + 1]}
    o_h, l_h = from_device(o)[b:b + 1, hs], from_device(lse)[b:b + 1, hs]
    del dev, dq, dk, dv, o, lse
    f = {x: si.as_f32(w, host[x]) for x in host}
    res = bwd_bounds.reference_and_bounds(f["q"][b:b + 1, hs], f["k"][b:b + 1, hk:hk + 1], f["v"][b:b + 1, hk:hk + 1],
                                          f["do"][b:b + 1, hs], o_h, l_h, w.scale, True, 0)
    bwd_bounds.check(got, res, f"{w.name} b={b} kv head {hk}")
