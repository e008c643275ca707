"""Pins of the float64 backward reference (CPU only).

The gradients are checked against things that do not use their formulas: central finite
differences of the forward reference's loss sum(dO * O), torch autograd on the CPU in float64
through an explicitly written masked softmax, and identities the chain rule forces (the dK rows
of a head sum to zero, the dV rows sum to the dO rows, a one-key head has dQ = dK = 0).  Broken
copies of the reference show that each plausible mistake is caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle

CASES = [(1, 1, 2, False, 0), (3, 5, 2, False, 0), (5, 3, 3, False, 0), (4, 4, 3, True, 0), (3, 7, 2, True, 4),
         (6, 4, 2, True, 0), (2, 6, 3, True, 0)]


def _rand(seed, nq, nk, d):
    g = np.random.default_rng(seed)
    return (g.standard_normal((nq, d)), g.standard_normal((nk, d)), g.standard_normal((nk, d)),
            g.standard_normal((nq, d)))


def check_finite_differences(bwd):
    """Central differences of L = sum(dO * O(q, k, v)) with the forward reference."""
    eps = 1e-5
    for seed, (nq, nk, d, causal, diag) in enumerate(CASES):
        q, k, v, do = _rand(10 + seed, nq, nk, d)
        scale = 0.8

        def loss(q_, k_, v_):
            o, _ = oracle.attention_head(q_, k_, v_, scale, causal, diag=diag)
            return float((o * do).sum())

        dq, dk, dv = bwd(q, k, v, do, scale, causal, diag)
        for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
                args_m = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert np.abs(num - g).max() < 1e-7, f"finite differences {name} case {seed}"


def check_torch_autograd(bwd):
    """torch autograd on the CPU in float64 through softmax(scale q k^T + mask) v."""
    for seed, (nq, nk, d, causal, diag) in enumerate([(16, 24, 8, False, 0), (20, 20, 8, True, 0),
                                                        (9, 30, 4, True, 21), (30, 9, 4, True, 0)]):
        q, k, v, do = _rand(50 + seed, nq, nk, d)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = 0.35 * tq @ tk.T
        if causal:
            s = s.masked_fill(~torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=diag), float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv
        (o * torch.tensor(do)).sum().backward()
        dq, dk, dv = bwd(q, k, v, do, 0.35, causal, diag)
        for name, a, b in (("dq", dq, tq.grad), ("dk", dk, tk.grad), ("dv", dv, tv.grad)):
            assert np.abs(a - b.numpy()).max() < 1e-10, f"torch autograd {name} case {seed}"


def check_identities(bwd):
    for seed, (nq, nk, d, causal, diag) in enumerate([(12, 17, 5, False, 0), (15, 15, 4, True, 0),
                                                        (6, 20, 3, True, 14)]):
        q, k, v, do = _rand(80 + seed, nq, nk, d)
        dq, dk, dv = bwd(q, k, v, do, 0.5, causal, diag)
        # every row's dS sums to zero, so the dK rows cancel; every row's P sums to one
        assert np.abs(dk.sum(axis=0)).max() < 1e-12, f"sum of dK rows, case {seed}"
        assert np.abs(dv.sum(axis=0) - do.sum(axis=0)).max() < 1e-12, f"sum of dV rows, case {seed}"
    q, k, v, do = _rand(90, 5, 1, 3)  # one key: P = 1, O = v_0, nothing depends on q or k
    dq, dk, dv = bwd(q, k, v, do, 0.5, False, 0)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    assert np.abs(dv[0] - do.sum(axis=0)).max() < 1e-13


CHECKS = [check_finite_differences, check_torch_autograd, check_identities]


def failures(bwd):
    out = []
    for c in CHECKS:
        try:
            c(bwd)
        except AssertionError as e:
            out.append(f"{c.__name__}: {e}")
    return out


def ref(q, k, v, do, scale, causal, diag):
    return oracle.attention_backward_head(q, k, v, do, scale, causal, diag)


def test_reference_passes_every_check():
    assert failures(ref) == []


def test_row_stat_equals_softmax_jacobian_term():
    q, k, v, do = _rand(3, 7, 9, 4)
    o, _ = oracle.attention_head(q, k, v, 0.6, False)
    p = oracle.attention_probs(q, k, 0.6)
    dp = do @ v.T
    assert np.abs(oracle.softmax_row_stat(o, do) - (p * dp).sum(axis=1)).max() < 1e-12


def test_grouped_heads_sum_over_their_query_heads():
    g = np.random.default_rng(4)
    B, H, Hkv, nq, nk, d = 1, 6, 2, 5, 7, 3
    q, do = g.standard_normal((B, H, nq, d)), g.standard_normal((B, H, nq, d))
    k, v = g.standard_normal((B, Hkv, nk, d)), g.standard_normal((B, Hkv, nk, d))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.4, True, nk - nq)
    rep = H // Hkv
    dq1, dk1, dv1 = oracle.attention_backward(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), do, 0.4, True,
                                              nk - nq)
    assert np.abs(dq - dq1).max() < 1e-13
    assert np.abs(dk - dk1.reshape(B, Hkv, rep, nk, d).sum(axis=2)).max() < 1e-12
    assert np.abs(dv - dv1.reshape(B, Hkv, rep, nk, d).sum(axis=2)).max() < 1e-12


def _broken(q, k, v, do, scale, causal, diag, *, mistake):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = scale * (q @ k.T)
    if causal:
        i = np.arange(s.shape[0])[:, None]
        j = np.arange(s.shape[1])[None, :]
        s = np.where(j > i + diag, -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    dv = (p.T @ do) if mistake != "dv_unnormalised" else (e.T @ do)
    dp = do @ v.T
    rs = (p * dp).sum(axis=1, keepdims=True)
    ds = {"row_term_dropped": p * dp, "row_term_sign": p * (dp + rs), "row_term_columns":
          p * (dp - (p * dp).sum(axis=0, keepdims=True)) if p.shape[0] == p.shape[1] else p * (dp - rs.mean())}.get(
        mistake, p * (dp - rs))
    dq = (1.0 if mistake == "dq_scale_dropped" else scale) * (ds @ k)
    dk = scale * ((ds.T @ q) if mistake != "dk_from_p" else (p.T @ q))
    if mistake == "dq_dk_swapped_scale":
        dq, dk = dq * scale, dk / scale
    return dq, dk, dv


MISTAKES = ["dv_unnormalised", "row_term_dropped", "row_term_sign", "row_term_columns", "dq_scale_dropped",
            "dk_from_p", "dq_dk_swapped_scale"]


def test_unbroken_copy_passes():
    assert failures(lambda *a: _broken(*a, mistake=None)) == []


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_mistake_is_caught(mistake):
    assert failures(lambda *a: _broken(*a, mistake=mistake)), f"{mistake} slipped through every check"
