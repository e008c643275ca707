"""The score-profile GPU tests can see the mistakes they are meant to catch (CPU only).

A float32 model of the kernels' online softmax (64-key tiles, the running max raised only when a
tile's max exceeds it by more than 8 log2 units, P rounded to bf16 for the P.V product, the bf16
rounding error of each tile's largest exponential added to the normaliser of O, O rounded to
bf16) is checked with the GPU tests' own tolerance check on the same profiles: the
faithful model passes on every profile, and each planted mistake in the rescale logic fails on
at least one profile.  Only the rising and late-spike profiles expose these mistakes (by
factors of 100 to 27000 over the tolerance); the falling and sawtooth ones never rescale after
their first tile.  The faithful model uses at most about half of the tolerance (the bf16
output rounding).  The same is shown for the backward's derived bounds (tests/bwd_bounds.py): a
float32 model of its arithmetic (P recomputed from the LSE, P and dS rounded to bf16, outputs
rounded to bf16) stays within the element-wise bound and the relative L2 bar on every profile,
and planted mistakes (the row term of dS dropped, dK without the scale, dQ from P instead of dS,
dV from dS instead of P, one 32 x 32 block of dS wrong in dK only, the causal mask one key too
wide) exceed them.  The models are test
infrastructure: the forward one follows the recurrence of the Day-21 page §5.2-5.3 with the
lazy threshold, the backward one the chain rule through the definition; neither is the oracle
or the GPU code."""
import math

import numpy as np
import pytest

import oracle
from synth import inputs as si
from synth.workloads import Workload
from tests.gpu_util import metrics
from tests.test_gpu_softmax_paths import PROFILES, SCALE, _inputs

TAU = 8.0
LOG2E = 1.0 / math.log(2.0)


def _bf16(x):
    return si.bf16_bits_to_f32(si.round_to_bf16_bits(np.asarray(x, np.float32)))


def _online_head(q, k, v, causal, mistake=None):
    """float32 online softmax over 64-key tiles for one head; returns (O as bf16 values, LSE)."""
    nq, nk = q.shape[0], k.shape[0]
    f32 = np.float32
    sl2 = f32(SCALE * LOG2E)
    m = np.full(nq, -np.inf, f32)
    l = np.zeros(nq, f32)
    c = np.zeros(nq, f32)  # bf16 rounding errors of the tiles' largest exponentials (normaliser of O only)
    acc = np.zeros((nq, v.shape[1]), f32)
    rows = np.arange(nq)
    for t0 in range(0, nk, 64):
        s = (q @ k[t0:t0 + 64].T).astype(f32)
        keys = np.arange(t0, min(t0 + 64, nk))
        if causal:
            s = np.where(keys[None, :] > rows[:, None], f32(-np.inf), s)
        mx = (s.max(axis=1) * sl2).astype(f32)
        m_old = m
        if np.any(mx > m + f32(TAU)):
            mnew = np.maximum(m, mx)
            if mistake == "alpha_sign":
                alpha = np.exp2(mnew - m).astype(f32)
                alpha = np.where(np.isfinite(alpha), alpha, f32(0))
            else:
                alpha = np.exp2(m - mnew).astype(f32)
            m = mnew.astype(f32)
            if mistake != "no_l_rescale":
                l = (l * alpha).astype(f32)
                c = (c * alpha).astype(f32)
            if mistake != "no_o_rescale":
                acc = (acc * alpha[:, None]).astype(f32)
        m_p = m_old if mistake == "p_uses_old_max" and t0 > 0 else m
        p = np.exp2(s * sl2 - m_p[:, None]).astype(f32)
        l = (l + p.sum(axis=1, dtype=f32)).astype(f32)
        pm = np.where(np.isfinite(mx), np.exp2(mx - m_p), 0).astype(f32)
        c = (c + (_bf16(pm) - pm)).astype(f32)
        acc = (acc + _bf16(p) @ v[t0:t0 + 64]).astype(f32)
    o = _bf16(acc / (l + c)[:, None])
    lse = ((m + np.log2(l)) / LOG2E).astype(f32)
    return o, lse


def _max_violation(kind, causal, mistake=None):
    """Largest ratio of an error metric to its bf16 tolerance (> 1 fails), over both heads."""
    from tests.gpu_util import BF16_LSE_MAXABS, BF16_O_MAXABS, BF16_O_RELL2

    nq, nk = (330, 330) if causal else (200, 330)
    q, k, v = (_bf16(a) for a in _inputs(kind, nq, nk, "bf16"))
    w = Workload("m", B=1, H=2, Nq=nq, Nk=nk, d=128, dtype="bf16", causal=causal, seed=5)
    o = np.empty((1, 2, nq, 128), np.float32)
    lse = np.empty((1, 2, nq), np.float32)
    for h in range(2):
        o[0, h], lse[0, h] = _online_head(q[0, h], k[0, h], v[0, h], causal, mistake)
    o_ref, l_ref = oracle.attention(q, k, v, SCALE, causal)
    mt = metrics(o, lse, o_ref, l_ref)
    if not mt["finite"]:
        return math.inf
    return max(mt["o_maxabs"] / BF16_O_MAXABS, mt["o_rel_l2"] / BF16_O_RELL2, mt["lse_maxabs"] / BF16_LSE_MAXABS)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", list(PROFILES))
def test_faithful_model_passes(kind, causal):
    assert _max_violation(kind, causal) <= 1.0


@pytest.mark.parametrize("mistake", ["no_o_rescale", "no_l_rescale", "alpha_sign", "p_uses_old_max"])
def test_planted_rescale_mistake_is_caught(mistake):
    worst = max(_max_violation(kind, causal, mistake) for kind in PROFILES for causal in (False, True))
    assert worst > 1.0, (mistake, worst)


def _backward_model(f, o_gpu, lse_gpu, causal, mistake=None):
    """The backward's arithmetic in float32 (scores and dP accumulated in fp32, P recomputed from the
    given LSE with exp2, dS = P (dP - Dr) in fp32, P and dS rounded to bf16 before the products,
    outputs rounded to bf16), optionally with one planted mistake; f holds [1, 2, N, d] float32
    arrays, o_gpu and lse_gpu the forward's outputs."""
    f32 = np.float32
    q, k, v, do = (f[x] for x in ("q", "k", "v", "do"))
    nq, nk = q.shape[2], k.shape[2]
    sl2 = f32(f32(SCALE) * f32(LOG2E))
    out = {x: np.zeros(f[y].shape, f32) for x, y in (("dq", "q"), ("dk", "k"), ("dv", "v"))}
    for h in range(q.shape[1]):
        s = (q[0, h] @ k[0, h].T).astype(f32)
        p = np.exp2((s * sl2 - (lse_gpu[0, h] * f32(LOG2E)).astype(f32)[:, None]).astype(f32)).astype(f32)
        if causal:
            lim = 1 if mistake == "mask_one_key_wide" else 0
            p = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None] + lim, p, f32(0))
        dp = (do[0, h] @ v[0, h].T).astype(f32)
        dr = (do[0, h] * o_gpu[0, h]).sum(axis=1, dtype=f32)
        row = f32(0) if mistake == "no_row_term" else dr[:, None]
        ds = (p * (dp - row).astype(f32)).astype(f32)
        dsb, pb = _bf16(ds), _bf16(p)
        ds_k = dsb.copy()
        if mistake == "one_block_of_dk" and h == 0:
            ds_k[64:96, 32:64] *= f32(1.25)
        sc_k = f32(1.0) if mistake == "dk_unscaled" else f32(SCALE)
        out["dq"][0, h] = _bf16(f32(SCALE) * ((pb if mistake == "dq_uses_p" else dsb) @ k[0, h]).astype(f32))
        out["dk"][0, h] = _bf16(sc_k * (ds_k.T @ q[0, h]).astype(f32))
        out["dv"][0, h] = _bf16(((dsb if mistake == "dv_uses_ds" else pb).T @ do[0, h]).astype(f32))
    return out


def _backward_violation(kind, causal, mistake=None):
    """Largest ratio, over dQ, dK and dV, of an element's error to its derived bound or of the
    relative L2 error to its derived bar (tests/bwd_bounds.py); <= 1 passes."""
    from tests import bwd_bounds

    nq, nk = (330, 330) if causal else (200, 330)
    q, k, v = _inputs(kind, nq, nk, "bf16")
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([5, 3])))
    do = g.standard_normal((1, 2, nq, 128)).astype(np.float32)
    f = {x: _bf16(a) for x, a in zip(("q", "k", "v", "do"), (q, k, v, do))}
    o, lse = oracle.attention(f["q"], f["k"], f["v"], SCALE, causal)
    o_gpu, lse_gpu = _bf16(o), lse.astype(np.float32)  # a forward's outputs: O in bf16, LSE in fp32
    got = _backward_model(f, o_gpu, lse_gpu, causal, mistake)
    res = bwd_bounds.reference_and_bounds(f["q"], f["k"], f["v"], f["do"], o_gpu, lse_gpu, SCALE, causal)
    worst = 0.0
    for x in ("dq", "dk", "dv"):
        ref, bound, pred = res[x]
        err = np.abs(got[x].astype(np.float64) - ref)
        rel = np.linalg.norm(got[x] - ref) / np.linalg.norm(ref)
        worst = max(worst, float((err / bound).max()), rel / (bwd_bounds.REL_L2_FACTOR * pred))
    return worst


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", list(PROFILES))
def test_backward_rounding_model_within_tolerance(kind, causal):
    assert _backward_violation(kind, causal) <= 1.0


@pytest.mark.parametrize("mistake", ["no_row_term", "dk_unscaled", "dq_uses_p", "dv_uses_ds", "one_block_of_dk",
                                     "mask_one_key_wide"])
def test_planted_backward_mistake_is_caught(mistake):
    worst = max(_backward_violation(kind, causal, mistake) for kind in PROFILES for causal in (False, True)
                if causal or mistake != "mask_one_key_wide")
    assert worst > 1.0, (mistake, worst)
