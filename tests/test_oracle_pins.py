"""Pins of the float64 reference implementation (CPU only).

The reference is checked against things other than itself: closed forms, invariants,
brute force, scipy/torch routines (tests/oracle_checks.py), the online recurrence written
from the Day-21 page §5.2-5.3 on tiny inputs, the Day-21 page's exercise 2 tolerance and the
Q31 answer's worked merge example (tests/golden/).  A set of deliberately broken copies of
the reference shows that each plausible mistake is caught by at least one check.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import recurrence
from tests import oracle_checks as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def ref_head(q, k, v, scale, causal):
    return oracle.attention_head(q, k, v, scale, causal)


def test_reference_passes_every_check():
    assert oc.failures(ref_head) == []


def test_reference_row_chunking_is_invisible():
    g = np.random.default_rng(0)
    q, k, v = g.standard_normal((37, 8)), g.standard_normal((37, 8)), g.standard_normal((37, 8))
    for causal in (False, True):
        o1, l1 = oracle.attention_head(q, k, v, 0.3, causal, row_chunk=1)
        o2, l2 = oracle.attention_head(q, k, v, 0.3, causal, row_chunk=1024)
        o3, l3 = oracle.attention_head(q, k, v, 0.3, causal, rows=np.arange(5, 30, 3))
        assert np.abs(o1 - o2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-13
        assert np.abs(o3 - o2[5:30:3]).max() < 1e-13 and np.abs(l3 - l2[5:30:3]).max() < 1e-13


def test_batched_equals_per_head():
    g = np.random.default_rng(1)
    q, k, v = (g.standard_normal((2, 3, 16, 4)) for _ in range(3))
    o, lse = oracle.attention(q, k, v, 0.5, True)
    for b in range(2):
        for h in range(3):
            o1, l1 = oracle.attention_head(q[b, h], k[b, h], v[b, h], 0.5, True)
            assert np.array_equal(o[b, h], o1) and np.array_equal(lse[b, h], l1)


def test_scores_and_probs_against_pure_python():
    """scores() and attention_probs() (no mask) against dot products and exponentials written out
    with Python loops and math.exp on a 5 x 7 head with d = 3; P's rows sum to one."""
    g = np.random.default_rng(3)
    q, k = g.standard_normal((5, 3)) * 2, g.standard_normal((7, 3)) * 2
    s = oracle.scores(q, k, 0.4)
    p = oracle.attention_probs(q, k, 0.4)
    for i in range(5):
        row = [0.4 * sum(q[i, c] * k[j, c] for c in range(3)) for j in range(7)]
        assert max(abs(a - b) for a, b in zip(row, s[i])) < 1e-14
        e = [math.exp(t) for t in row]
        assert max(abs(a / sum(e) - b) for a, b in zip(e, p[i])) < 1e-15
        assert abs(p[i].sum() - 1.0) < 1e-14


# ---------------------------------------------------------------- planted mistakes
def _variant(q, k, v, scale, causal, *, mistake):
    """A copy of the reference's steps with one planted mistake."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    sc = 1.0 if mistake == "scale_ignored" else (scale * scale if mistake == "scale_squared" else scale)
    s = sc * (q @ k.T)
    i = np.arange(s.shape[0])[:, None]
    j = np.arange(s.shape[1])[None, :]
    if causal:
        masked = {"mask_flipped": j < i, "mask_diagonal": j >= i}.get(mistake, j > i)
        s = np.where(masked, -np.inf, s)
    axis = 0 if mistake == "softmax_over_queries" else 1
    m = s.max(axis=axis, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=axis, keepdims=True)
    p = e if mistake == "no_normalisation" else e / l
    vv = v[::-1] if mistake == "v_rows_reversed" else v
    o = (p.T if mistake == "p_transposed" else p) @ vv
    mm, ll = m.reshape(-1), l.reshape(-1)
    if mistake == "lse_log2":
        lse = mm + np.log2(ll)
    elif mistake == "lse_without_max":
        lse = np.log(ll)
    elif mistake == "lse_sign":
        lse = mm - np.log(ll)
    else:
        lse = mm + np.log(ll)
    return o, lse


MISTAKES = ["scale_ignored", "scale_squared", "mask_flipped", "mask_diagonal", "softmax_over_queries",
            "no_normalisation", "v_rows_reversed", "p_transposed", "lse_log2", "lse_without_max",
            "lse_sign"]


def test_unbroken_variant_passes():
    assert oc.failures(lambda *a: _variant(*a, mistake=None)) == []


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_mistake_is_caught(mistake):
    assert oc.failures(lambda *a: _variant(*a, mistake=mistake)), f"{mistake} slipped through every check"


# ---------------------------------------------------------------- online recurrence (Day-21 §5.2-5.3)
def test_recurrence_equals_two_pass_brute_force_grid():
    g = np.random.default_rng(2)
    for nk in range(1, 18):
        for d in (1, 4):
            q = g.standard_normal(d)
            k = g.standard_normal((nk, d)) * 3.0
            v = g.standard_normal((nk, d))
            o_ref, l_ref = oracle.attention_head(q[None], k, v, 0.7, False)
            for block in sorted({1, 2, 3, 4, nk}):
                o, lse = recurrence.attention_row(q.tolist(), k.tolist(), v.tolist(), 0.7, block)
                assert np.abs(np.array(o) - o_ref[0]).max() < 1e-12
                assert abs(lse - l_ref[0]) < 1e-12


def test_day21_exercise_online_softmax():
    """The exercise's vector softmax, block by block: one query q = [1] against keys [x_j] with
    one-hot value rows, so the recurrence's output row is softmax(x) itself."""
    ex = _golden("day21_online_softmax_exercise.json")
    x = np.random.default_rng(ex["seed"]).standard_normal(ex["n"]) * ex["std"]
    n = len(x)
    one_hot = [[1.0 if r == c else 0.0 for c in range(n)] for r in range(n)]
    online, lse = recurrence.attention_row([1.0], [[t] for t in x], one_hot, 1.0, ex["block"])
    p, m, l = oracle.softmax_two_pass(x[None])
    err = np.abs(np.array(online) - p[0]).max()
    assert err < ex["tolerance"]  # the page's bound
    assert err < 1e-15            # in float64 the two agree to rounding
    assert abs(sum(online) - 1.0) < 1e-12
    assert abs(lse - (m[0] + math.log(l[0]))) < 1e-12


def test_q31_worked_merge_example():
    """Blocks with maxima 10 and 12 merge by rescaling the first by exp(10 - 12)."""
    ex = _golden("q31_block_merge.json")
    m1, m2 = ex["block1_max"], ex["block2_max"]
    x = [m1, m1 - 1.0, m2, m2 - 1.0]  # block 1 = [10, 9], block 2 = [12, 11]
    eye = [[1.0 if r == c else 0.0 for c in range(4)] for r in range(4)]
    # States of the two blocks; with q = 1 (d = 1), keys x, values = identity rows, O equals P.
    s1 = recurrence.partial_state([1.0], [[x[0]], [x[1]]], eye[:2], 1.0)
    s2 = recurrence.partial_state([1.0], [[x[2]], [x[3]]], eye[2:], 1.0)
    assert s1[0] == m1 and s2[0] == m2
    m, l, acc = recurrence.merge_states(s1, s2)
    factor = math.exp(ex["rescale_exponent"])
    assert m == m2
    assert abs(l - (factor * s1[1] + s2[1])) < 1e-15
    assert abs(l - (1 + math.exp(-1)) * (1 + math.exp(-2))) < 1e-14
    two_pass = sum(math.exp(t - m2) for t in x)
    assert abs(l - two_pass) < 1e-14
    o, lse = recurrence.finish((m, l, acc))
    p_closed = [math.exp(t - m2) / two_pass for t in x]
    assert max(abs(a - b) for a, b in zip(o, p_closed)) < 1e-15
    assert abs(lse - (m2 + math.log(two_pass))) < 1e-14
    # the same two blocks as two decode splits, merged by the reference's combine
    o_s = np.array([acc_i for acc_i in (s1[2], s2[2])])
    oc_, lc = oracle.combine_partials(o_s, np.array([s1[0], s2[0]]), np.array([s1[1], s2[1]]))
    assert np.abs(oc_ - np.array(p_closed)).max() < 1e-15 and abs(lc - lse) < 1e-14


# ---------------------------------------------------------------- split-KV partials and combine
@pytest.mark.parametrize("nk,splits", [(1, 1), (7, 1), (7, 2), (7, 7), (64, 64), (100, 64), (1000, 64),
                                       (513, 4), (10, 3)])
def test_split_combine_partition_invariance(nk, splits):
    g = np.random.default_rng(nk * 131 + splits)
    d = 8
    q = g.standard_normal(d)
    k = g.standard_normal((nk, d)) * 2.0
    v = g.standard_normal((nk, d))
    o_ref, l_ref = oracle.attention_head(q[None], k, v, 0.35, False)
    o_s, m_s, l_s = oracle.split_partials(q, k, v, 0.35, splits)
    o, lse = oracle.combine_partials(o_s, m_s, l_s)
    assert np.abs(o - o_ref[0]).max() < 1e-12 and abs(lse - l_ref[0]) < 1e-12
    # each split's state equals the pure-Python chunk state
    for s, (a, b) in enumerate(oracle.split_bounds(nk, splits)):
        m, l, acc = recurrence.partial_state(q.tolist(), k[a:b].tolist(), v[a:b].tolist(), 0.35)
        assert (m == m_s[s] == -math.inf) or abs(m - m_s[s]) < 1e-12
        assert abs(l - l_s[s]) < 1e-12 and np.abs(np.array(acc) - o_s[s]).max() < 1e-12


def test_split_bounds_cover_keys_once():
    for nk in (1, 5, 64, 100, 32768):
        for s in (1, 3, 64):
            if s > nk:
                continue
            b = oracle.split_bounds(nk, s)
            covered = [j for a, e in b for j in range(a, e)]
            assert covered == list(range(nk))
            assert b[0][1] > b[0][0]  # the first split is never empty


def test_combine_ignores_empty_splits():
    g = np.random.default_rng(3)
    o_s = g.standard_normal((4, 5))
    m_s = np.array([1.0, -np.inf, 3.0, -np.inf])
    l_s = np.array([2.0, 0.0, 1.5, 0.0])
    o_s[1] = o_s[3] = 0.0
    o, lse = oracle.combine_partials(o_s, m_s, l_s)
    o2, l2 = oracle.combine_partials(o_s[[0, 2]], m_s[[0, 2]], l_s[[0, 2]])
    assert np.abs(o - o2).max() == 0.0 and lse == l2
