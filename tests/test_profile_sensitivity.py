"""The score-profile GPU tests can see the mistakes they are meant to catch (CPU only).

A float32 model of the kernels' online softmax (64-key tiles, the running max raised only when a
tile's max exceeds it by more than 8 log2 units, P rounded to bf16 for the P.V product, O
rounded to bf16) is checked with the GPU tests' own tolerance check on the same profiles: the
faithful model passes on every profile, and each planted mistake in the rescale logic fails on
at least one profile.  Only the rising and late-spike profiles expose these mistakes (by
factors of 100 to 27000 over the tolerance); the falling and sawtooth ones never rescale after
their first tile.  The faithful model uses at most about half of the tolerance (the bf16
output rounding).  The same is shown for the backward's derived tolerance: a model with its
bf16 roundings of P, dS and the outputs stays within it on every profile (at most about half),
and planted mistakes (the row term of dS dropped, dK without the scale, dQ from P instead of
dS, dV from dS instead of P) exceed it by factors of 35 and more.  The models are test
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
            if mistake != "no_o_rescale":
                acc = (acc * alpha[:, None]).astype(f32)
        m_p = m_old if mistake == "p_uses_old_max" and t0 > 0 else m
        p = np.exp2(s * sl2 - m_p[:, None]).astype(f32)
        l = (l + p.sum(axis=1, dtype=f32)).astype(f32)
        acc = (acc + _bf16(p) @ v[t0:t0 + 64]).astype(f32)
    o = _bf16(acc / l[:, None])
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


def _backward_model(f, causal, mistake=None):
    """float64 gradients with the backward's roundings (P and dS to bf16 before their products,
    outputs to bf16), optionally with one planted mistake; f holds [1, 2, N, d] float32 arrays."""
    q, k, v, do = (f[x][0].astype(np.float64) for x in ("q", "k", "v", "do"))
    s = SCALE * q @ k.transpose(0, 2, 1)
    if causal:
        s = np.where(np.arange(k.shape[1])[None, None, :] > np.arange(q.shape[1])[None, :, None], -np.inf, s)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    o = _bf16(p @ v).astype(np.float64)
    row = (do * o).sum(-1, keepdims=True)
    ds = p * (do @ v.transpose(0, 2, 1) - (0.0 if mistake == "no_row_term" else row))
    pb, dsb = _bf16(p).astype(np.float64), _bf16(ds).astype(np.float64)
    sc_k = 1.0 if mistake == "dk_unscaled" else SCALE
    dq = _bf16(SCALE * (pb if mistake == "dq_uses_p" else dsb) @ k)
    dk = _bf16(sc_k * dsb.transpose(0, 2, 1) @ q)
    dv = _bf16((dsb if mistake == "dv_uses_ds" else pb).transpose(0, 2, 1) @ do)
    return {"dq": dq, "dk": dk, "dv": dv}


def _backward_violation(kind, causal, mistake=None):
    from tests.test_gpu_bwd import _rel_l2
    from tests.test_gpu_softmax_paths import _backward_tolerances

    nq, nk = (330, 330) if causal else (200, 330)
    q, k, v = _inputs(kind, nq, nk, "bf16")
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([5, 3])))
    do = g.standard_normal((1, 2, nq, 128)).astype(np.float32)
    f = {x: _bf16(a) for x, a in zip(("q", "k", "v", "do"), (q, k, v, do))}
    got = _backward_model(f, causal, mistake)
    ref = dict(zip(("dq", "dk", "dv"), oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], SCALE, causal)))
    tol = _backward_tolerances(f, causal)
    return max(_rel_l2(got[x][None], ref[x]) / tol[x] for x in tol)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", list(PROFILES))
def test_backward_rounding_model_within_tolerance(kind, causal):
    assert _backward_violation(kind, causal) <= 1.0


@pytest.mark.parametrize("mistake", ["no_row_term", "dk_unscaled", "dq_uses_p", "dv_uses_ds"])
def test_planted_backward_mistake_is_caught(mistake):
    worst = max(_backward_violation(kind, causal, mistake) for kind in PROFILES for causal in (False, True))
    assert worst > 1.0, (mistake, worst)
