"""Pins of the float64 reference's arbitrary element mask (CPU only).

The mask is a boolean matrix allowed [Nq, Nk]: key j is visible to query row i iff allowed[i, j]
(the rule of the Day-21 page's §6 table: skip blocks that are masked out, mask partial blocks
element by element; the Q31 answer §2 names arbitrary masks as what FlashAttention-2 lacks).
A row with no visible key has O = 0 and LSE = -inf.  The reference is checked against:
  * a pure-Python brute force of the textbook softmax over the visible keys of each row;
  * torch's scaled_dot_product_attention on the CPU in float64 with the same boolean mask (rows
    with at least one visible key);
  * the masks it must reduce to: all true (no mask), the causal lower triangle with any diagonal
    offset (the reference's own causal path, itself pinned in test_oracle_pins_masks_gqa.py);
  * invariance under permuting the keys together with V's rows and the mask's columns;
  * the empty-row convention, and a row with one visible key (O = that key's V row, LSE = its score).
Broken copies show that plausible mistakes (mask transposed, inverted, ignored, applied after the
normalisation, empty rows left as NaN) are each caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle

TOL = 1e-12


def _head(seed, nq, nk, d):
    g = np.random.default_rng(seed)
    return g.standard_normal((nq, d)), g.standard_normal((nk, d)) * 1.5, g.standard_normal((nk, d))


def _mask(seed, nq, nk, p=0.5, empty_rows=()):
    m = np.random.default_rng(seed).random((nq, nk)) < p
    for r in empty_rows:
        m[r] = False
    return m


def brute_force_masked(q, k, v, scale, allowed):
    nq, dv = len(q), len(v[0])
    o = np.zeros((nq, dv))
    lse = np.zeros(nq)
    for i in range(nq):
        vis = [j for j in range(len(k)) if allowed[i][j]]
        if not vis:
            lse[i] = -math.inf
            continue
        e = {j: math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j]))) for j in vis}
        den = math.fsum(e.values())
        for c in range(dv):
            o[i, c] = math.fsum(e[j] * float(v[j][c]) for j in vis) / den
        lse[i] = math.log(den)
    return o, lse


# ------------------------------------------------------------- checks on a masked one-head function
def check_brute_force(attn):
    for seed, (nq, nk, d) in enumerate([(1, 1, 2), (3, 7, 3), (9, 5, 4), (12, 12, 2), (6, 20, 3)]):
        q, k, v = _head(500 + seed, nq, nk, d)
        m = _mask(600 + seed, nq, nk, 0.6, empty_rows=(nq - 1,) if nq > 2 else ())
        o, lse = attn(q, k, v, 0.7, m)
        ob, lb = brute_force_masked(q.tolist(), k.tolist(), v.tolist(), 0.7, m.tolist())
        assert np.abs(o - ob).max() < TOL, "brute force O"
        assert np.array_equal(np.isneginf(lse), np.isneginf(lb)), "empty rows"
        fin = np.isfinite(lb)
        assert np.abs(lse[fin] - lb[fin]).max() < TOL, "brute force LSE"


def check_torch_sdpa(attn):
    for seed, (nq, nk, d) in enumerate([(8, 8, 4), (5, 30, 8), (33, 17, 6)]):
        q, k, v = _head(700 + seed, nq, nk, d)
        m = _mask(800 + seed, nq, nk, 0.3)
        m[:, seed] = True  # every row keeps at least one key: torch's output for an empty row is not defined here
        o, _ = attn(q, k, v, 0.4, m)
        ot = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            attn_mask=torch.from_numpy(m)[None], scale=0.4)[0].numpy()
        assert np.abs(o - ot).max() < 1e-10, "torch SDPA with a boolean mask"


def check_reductions(attn):
    q, k, v = _head(900, 14, 14, 5)
    o, lse = attn(q, k, v, 0.5, np.ones((14, 14), bool))
    o0, l0 = oracle.attention_head(q, k, v, 0.5, False)
    assert np.abs(o - o0).max() < TOL and np.abs(lse - l0).max() < TOL, "all-true mask = no mask"
    for nq, nk, diag in [(14, 14, 0), (6, 14, 8), (14, 9, 0)]:
        qq, kk, vv = q[:nq], k[:nk], v[:nk]
        tri = np.arange(nk)[None, :] <= np.arange(nq)[:, None] + diag
        o, lse = attn(qq, kk, vv, 0.5, tri)
        oc, lc = oracle.attention_head(qq, kk, vv, 0.5, True, diag=diag)
        assert np.abs(o - oc).max() < TOL and np.abs(lse - lc).max() < TOL, "triangle mask = causal"


def check_key_permutation(attn):
    q, k, v = _head(901, 10, 25, 4)
    m = _mask(902, 10, 25, 0.4)
    perm = np.random.default_rng(903).permutation(25)
    o, lse = attn(q, k, v, 0.8, m)
    op, lp = attn(q, k[perm], v[perm], 0.8, m[:, perm])
    fin = np.isfinite(lse)
    assert np.abs(o - op).max() < TOL and np.abs(lse[fin] - lp[fin]).max() < TOL, "key permutation"


def check_special_rows(attn):
    q, k, v = _head(904, 4, 6, 3)
    m = np.zeros((4, 6), bool)
    m[1, 4] = True                      # one visible key
    m[2, :] = True                      # all keys
    m[3, [0, 5]] = True
    o, lse = attn(q, k, v, 0.9, m)
    assert np.all(o[0] == 0.0) and np.isneginf(lse[0]), "empty row: O = 0, LSE = -inf"
    assert np.abs(o[1] - v[4]).max() < TOL, "one visible key: O = its V row"
    assert abs(lse[1] - 0.9 * float(q[1] @ k[4])) < TOL, "one visible key: LSE = its score"
    assert np.isfinite(o).all()


CHECKS = [check_brute_force, check_torch_sdpa, check_reductions, check_key_permutation, check_special_rows]


def failures(attn):
    out = []
    for c in CHECKS:
        try:
            c(attn)
        except AssertionError as e:
            out.append(f"{c.__name__}: {e}")
    return out


def ref(q, k, v, scale, allowed):
    return oracle.attention_head(q, k, v, scale, allowed=allowed)


def test_reference_passes_every_check():
    assert failures(ref) == []


def test_batched_mask_is_shared_by_every_head():
    g = np.random.default_rng(905)
    q, k, v = (g.standard_normal((2, 3, 9, 4)) for _ in range(3))
    m = _mask(906, 9, 9, 0.5, empty_rows=(2,))
    o, lse = oracle.attention(q, k, v, 0.5, allowed=m)
    for b in range(2):
        for h in range(3):
            o1, l1 = oracle.attention_head(q[b, h], k[b, h], v[b, h], 0.5, allowed=m)
            assert np.array_equal(o[b, h], o1) and np.array_equal(lse[b, h], l1)


def test_rows_argument_uses_true_row_index():
    q, k, v = _head(907, 20, 30, 4)
    m = _mask(908, 20, 30, 0.5, empty_rows=(7,))
    o, lse = oracle.attention_head(q, k, v, 0.6, allowed=m)
    rows = np.array([0, 7, 13, 19])
    o2, l2 = oracle.attention_head(q, k, v, 0.6, allowed=m, rows=rows)
    assert np.array_equal(o2, o[rows]) and np.array_equal(np.isneginf(l2), np.isneginf(lse[rows]))


def _broken(q, k, v, scale, allowed, *, mistake):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    m = np.asarray(allowed, bool)
    if mistake == "transposed" and m.shape[0] == m.shape[1]:
        m = m.T
    elif mistake == "transposed":
        m = np.resize(m.T, m.shape)
    elif mistake == "inverted":
        m = ~m
    elif mistake == "first_row_unmasked":
        m = m.copy()
        m[0] = True
    s = scale * q @ k.T
    if mistake == "after_normalisation":
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True) * m
        o = p @ v
        with np.errstate(divide="ignore"):
            lse = np.where(m.any(axis=1), np.log((np.exp(s) * m).sum(axis=1)), -np.inf)
        return o, lse
    s = np.where(m, s, -np.inf)
    with np.errstate(invalid="ignore"):
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        l = e.sum(axis=1, keepdims=True)
        o = (e / l) @ v
        lse = mx[:, 0] + np.log(l[:, 0])
    if mistake != "empty_rows_nan":
        empty = ~m.any(axis=1)
        o[empty] = 0.0
        lse[empty] = -np.inf
    return o, lse


MISTAKES = ["transposed", "inverted", "first_row_unmasked", "after_normalisation", "empty_rows_nan"]


def test_unbroken_copy_passes():
    assert failures(lambda *a: _broken(*a, mistake=None)) == []


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_mask_mistake_is_caught(mistake):
    assert failures(lambda *a: _broken(*a, mistake=mistake)), f"{mistake} slipped through every check"
