"""Parity of the forward kernels with the float64 reference on score profiles built to drive
every branch of the online softmax (Day-21 page §5.2-5.3: the running max, the rescale of the
running sum and of the accumulator when the max grows, the exponentials taken against a max
that is allowed to lag behind).

Every query has the same large first component and K's first component follows a chosen
profile along the keys, so each row of scores is that profile (in log2 units below) plus a
small seeded noise:
  * rising_fast: +10 per 64-key tile, above the kernels' lazy-rescale thresholds (8 for bf16 and
    fp32 inputs, 4 for FP8), so the running max and the accumulators are rescaled on every tile;
  * rising_slow: +3 per tile, below them: the max used for the exponentials lags the true
    one, the exponentials exceed 1, and the rescale fires only every few tiles;
  * falling: the max sits in the first tile and never moves afterwards;
  * sawtooth: +12 across each tile, back to 0 at the next tile's first key;
  * late_spike: flat, with the last key (in a ragged last tile) 30 above the rest.
With fp32 inputs the Q and K noise is left out: the scores reach hundreds of log2 units, and
fp32 rounding of a dot product that adds small terms to one large one would otherwise be of the
size of the fp32 tolerance by itself; without it every q.k is exact in fp32.
The other head of each case is plain noise.  Tolerances are the suite's: the bf16 and fp32
bounds of the forward tests, for FP8 inputs the element-wise bound derived in the FP8 forward
tests, and for the backward the bounds derived from its arithmetic in tests/bwd_bounds.py."""
import math

import numpy as np
import pytest
import torch

import exact_attention_126_amd as fa
import oracle
from synth import inputs as si
from synth.workloads import Workload
from tests import bwd_bounds
from tests.gpu_util import assert_parity, from_device, metrics, to_device
from tests.test_gpu_fp8_fwd import _check as fp8_check

pytestmark = pytest.mark.gpu

PROFILES = {
    "rising_fast": lambda j, n: 10.0 * j / 64,
    "rising_slow": lambda j, n: 3.0 * j / 64,
    "falling": lambda j, n: -10.0 * j / 64,
    "sawtooth": lambda j, n: 12.0 * (j % 64) / 64,
    "late_spike": lambda j, n: np.where(j == n - 1, 30.0, 0.0),
}
D = 128
SCALE = 1.0 / math.sqrt(D)


def _profile_head(kind, Nq, Nk, seed, noise):
    """float32 Q, K, V of one head whose scores are PROFILES[kind] (log2 units) plus noise."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    q = (noise * g.standard_normal((Nq, D))).astype(np.float32)
    k = (noise * g.standard_normal((Nk, D))).astype(np.float32)
    v = g.standard_normal((Nk, D)).astype(np.float32)
    q[:, 0] = 4.0
    k[:, 0] = PROFILES[kind](np.arange(Nk), Nk) * math.log(2.0) / (4.0 * SCALE)
    return q, k, v


def _noise_head(Nq, Nk, seed):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2])))
    return tuple(g.standard_normal((n, D)).astype(np.float32) for n in (Nq, Nk, Nk))


def _inputs(kind, Nq, Nk, dtype, seed=5):
    """[1, 2, N, D] float32 Q, K, V: head 0 the profile, head 1 noise."""
    heads = [_profile_head(kind, Nq, Nk, seed, 0.0 if dtype == "f32" else 0.1), _noise_head(Nq, Nk, seed)]
    return tuple(np.stack([h[i] for h in heads])[None] for i in range(3))


CASES = [(kind, dtype, causal, n)
         for kind in PROFILES
         for dtype, causal, n in [("bf16", False, (200, 330)), ("bf16", True, (330, 330)), ("f32", False, (70, 330))]]


@pytest.mark.parametrize("kind,dtype,causal,shape", CASES,
                         ids=[f"{c[0]}_{c[1]}{'_causal' if c[2] else ''}" for c in CASES])
def test_profile_matches_reference(kind, dtype, causal, shape):
    Nq, Nk = shape
    q, k, v = _inputs(kind, Nq, Nk, dtype)
    w = Workload(f"{kind}_{dtype}", B=1, H=2, Nq=Nq, Nk=Nk, d=D, dtype=dtype, causal=causal, seed=5)
    store = (lambda x: si.round_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    host = {"q": store(q), "k": store(k), "v": store(v)}
    print(f"  [fa_fwd] profile {kind}: Nq={Nq} Nk={Nk} d={D} {dtype} causal={causal}", flush=True)
    o, lse = fa.attention(*(to_device(w, host[x]) for x in "qkv"), causal=causal, scale=SCALE)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(*(si.as_f32(w, host[x]) for x in "qkv"), SCALE, causal)
    assert_parity(dtype, metrics(from_device(o), from_device(lse), o_ref, l_ref), f"{kind} {dtype}")


def _to_e4m3(x):
    """[rows, d] float32 -> (E4M3 codes, scale) with scale = max|x| / 448, the suite's FP8 recipe."""
    amax = float(np.abs(x).max())
    scale = np.float32(amax / si.E4M3_MAX)
    y = np.clip(x / scale, -si.E4M3_MAX, si.E4M3_MAX).astype(np.float32)
    return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy(), scale


@pytest.mark.parametrize("kind", list(PROFILES))
@pytest.mark.parametrize("align", [None, "top_left"])
def test_profile_fp8_matches_reference(kind, align):
    Nq, Nk = (330, 330) if align else (200, 330)
    x = dict(zip("qkv", _inputs(kind, Nq, Nk, "e4m3")))
    w = Workload(f"{kind}_fp8", B=1, H=2, H_kv=2, Nq=Nq, Nk=Nk, d=D, dtype="bf16", causal=align is not None, seed=5,
                 causal_align=align or "top_left", kv_dtype="e4m3", q_dtype="e4m3")
    host, dev = {}, {}
    for t in "qkv":
        codes = np.empty(x[t].shape, np.uint8)
        scales = np.empty((1, 2), np.float32)
        for h in range(2):
            codes[0, h], scales[0, h] = _to_e4m3(x[t][0, h])
        host[t], host[t + "s"] = codes, scales
        dev[t], dev[t + "s"] = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    mask = fa.FA_MASK_CAUSAL if align else fa.FA_MASK_NONE
    print(f"  [fa_fwd_fp8] profile {kind}: Nq={Nq} Nk={Nk} d={D} mask={align}", flush=True)
    o, lse = fa.attention_fp8(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], dev["vs"], mask, SCALE)
    torch.cuda.synchronize()
    fp8_check(w, host, o, lse, [(0, 0), (0, 1)])


@pytest.mark.parametrize("kind", list(PROFILES))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_profile_decode_matches_reference(kind, dtype):
    """Split-KV decode over 1500 keys in 3 splits of 500 (ragged against the kernel's 64-row
    steps): the split kernel's running max moves on every step for the rising profiles, and the
    combine merges splits whose maxima differ by up to ~80 log2 units."""
    Nk, S = 1500, 3
    q, k, v = _inputs(kind, 1, Nk, dtype)
    w = Workload(f"{kind}_decode_{dtype}", B=1, H=2, Nq=1, Nk=Nk, d=D, dtype=dtype, causal=False, seed=5)
    store = (lambda x: si.round_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    host = {"q": store(q), "k": store(k), "v": store(v)}
    print(f"  [fa_decode] profile {kind}: Nk={Nk} splits={S} d={D} {dtype}", flush=True)
    o, lse = fa.decode(*(to_device(w, host[x]) for x in "qkv"), S, scale=SCALE)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(*(si.as_f32(w, host[x]) for x in "qkv"), SCALE, False)
    assert_parity(dtype, metrics(from_device(o), from_device(lse), o_ref, l_ref), f"decode {kind} {dtype}")


@pytest.mark.parametrize("kind", list(PROFILES))
@pytest.mark.parametrize("align", [None, "top_left"])
def test_profile_backward_matches_reference(kind, align):
    """fa_bwd on the GPU forward's O and LSE for the same profiles, against the reference
    gradients of the plain definition, within the element-wise bounds and the relative L2 bars
    derived from the backward's arithmetic (tests/bwd_bounds.py).  On these profiles K and Q carry
    one component near 100 while the gradient cancels in it, so rounding dS to bf16 costs dQ far
    more than on random inputs; the derived bounds follow that."""
    Nq, Nk = (330, 330) if align else (200, 330)
    q, k, v = _inputs(kind, Nq, Nk, "bf16")
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([5, 3])))
    do = g.standard_normal((1, 2, Nq, D)).astype(np.float32)
    w = Workload(f"{kind}_bwd", B=1, H=2, Nq=Nq, Nk=Nk, d=D, dtype="bf16", causal=align is not None, seed=5)
    host = {x: si.round_to_bf16_bits(a) for x, a in zip(("q", "k", "v", "do"), (q, k, v, do))}
    dev = {x: to_device(w, host[x]) for x in host}
    mask = fa.FA_MASK_CAUSAL if align else fa.FA_MASK_NONE
    print(f"  [fa_fwd_ex + fa_bwd] profile {kind}: Nq={Nq} Nk={Nk} d={D} mask={align}", flush=True)
    o = torch.empty_like(dev["q"])
    lse = torch.empty((1, 2, Nq), dtype=torch.float32, device="cuda")
    fa.fa_fwd_ex(dev["q"], dev["k"], dev["v"], o, lse, mask, SCALE)
    dq, dk, dv = fa.attention_backward(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale=SCALE, mask=mask)
    torch.cuda.synchronize()
    f = {x: si.as_f32(w, host[x]) for x in host}
    res = bwd_bounds.reference_and_bounds(f["q"], f["k"], f["v"], f["do"], from_device(o), from_device(lse), SCALE,
                                          align is not None)
    rq, rk, rv = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], SCALE, align is not None)
    for x, r in (("dq", rq), ("dk", rk), ("dv", rv)):
        assert np.abs(res[x][0] - r).max() <= 1e-9 * max(1.0, np.abs(r).max())
    bwd_bounds.check({"dq": from_device(dq), "dk": from_device(dk), "dv": from_device(dv)}, res,
                     f"profile {kind} mask={align}")
