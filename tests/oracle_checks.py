"""Checks that pin the reference implementation to what the pages and the mathematics fix.

Each check takes an implementation `attn(q, k, v, scale, causal) -> (O, LSE)` of one head
(float64 numpy arrays) and raises AssertionError when it is violated.  The pin tests run
them against the reference implementation (all must pass) and against deliberately broken
copies of it (each must be caught by at least one check).

None of these checks retypes the reference's formula: they compare against closed forms,
invariants, a brute-force evaluation of the textbook softmax definition, library routines,
and the pages' worked example.
"""
from __future__ import annotations

import math

import numpy as np

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_head(seed, nq, nk, d, scale_k=1.0):
    g = _rng(seed)
    return g.standard_normal((nq, d)), g.standard_normal((nk, d)) * scale_k, g.standard_normal((nk, d))


# --- brute force: the textbook definition softmax(x)_i = e^{x_i} / sum_j e^{x_j}, no max trick,
#     exact summation (math.fsum), pure Python.  Only for small, well-scaled inputs.
def brute_force_head(q, k, v, scale, causal):
    nq, nk, dv = len(q), len(k), len(v[0])
    o = [[0.0] * dv for _ in range(nq)]
    lse = [0.0] * nq
    for i in range(nq):
        allowed = [j for j in range(nk) if not (causal and j > i)]
        e = {j: math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j]))) for j in allowed}
        den = math.fsum(e.values())
        for c in range(dv):
            o[i][c] = math.fsum(e[j] * float(v[j][c]) for j in allowed) / den
        lse[i] = math.log(den)
    return np.array(o), np.array(lse)


def check_brute_force(attn):
    for seed, (nq, nk, d) in enumerate([(1, 1, 1), (3, 5, 2), (7, 7, 4), (6, 9, 3), (16, 16, 8)]):
        q, k, v = _rand_head(100 + seed, nq, nk, d)
        for causal in ([False, True] if nq == nk else [False]):
            o, lse = attn(q, k, v, 1.0 / math.sqrt(d), causal)
            ob, lb = brute_force_head(q.tolist(), k.tolist(), v.tolist(), 1.0 / math.sqrt(d), causal)
            assert np.abs(o - ob).max() < 1e-12, "brute force O"
            assert np.abs(lse - lb).max() < 1e-12, "brute force LSE"


def check_constant_v(attn):
    """V rows all equal to c  =>  every O row equals c (weights sum to one)."""
    q, k, _ = _rand_head(1, 24, 40, 8)
    c = _rng(2).standard_normal(8)
    v = np.tile(c, (40, 1))
    o, _ = attn(q, k, v, 0.3, False)
    assert np.abs(o - c).max() < TOL, "constant V"
    q, k, _ = _rand_head(3, 24, 24, 8)
    o, _ = attn(q, k, np.tile(c, (24, 1)), 0.3, True)
    assert np.abs(o - c).max() < TOL, "constant V causal"


def check_one_hot_rowsum(attn):
    """V_j = e_j (identity, Nk = dv) => O equals P: rows sum to 1, entries >= 0, causal zeros above diagonal."""
    n = 12
    q, k, _ = _rand_head(4, n, n, 5)
    for causal in (False, True):
        p, _ = attn(q, k, np.eye(n), 0.7, causal)
        assert np.abs(p.sum(axis=1) - 1).max() < TOL, "P rows sum to 1"
        assert p.min() >= 0, "P >= 0"
        if causal:
            assert np.abs(np.triu(p, 1)).max() == 0.0, "causal: no weight on keys after the query"
        else:
            assert p[np.triu_indices(n, 1)].min() > 0, "non-causal: every key gets weight"


def check_permutation_invariance(attn):
    """Permuting K and V rows together leaves O and LSE unchanged (non-causal)."""
    q, k, v = _rand_head(5, 10, 33, 6)
    perm = _rng(6).permutation(33)
    o1, l1 = attn(q, k, v, 0.5, False)
    o2, l2 = attn(q, k[perm], v[perm], 0.5, False)
    assert np.abs(o1 - o2).max() < TOL and np.abs(l1 - l2).max() < TOL, "K/V joint permutation"


def check_zero_query(attn):
    """Q = 0 => uniform weights: O_i = mean of the allowed V rows, LSE_i = ln(#allowed)."""
    n, d = 19, 4
    _, k, v = _rand_head(7, n, n, d)
    q = np.zeros((n, d))
    o, lse = attn(q, k, v, 0.25, False)
    assert np.abs(o - v.mean(axis=0)).max() < TOL, "Q=0 mean"
    assert np.abs(lse - math.log(n)).max() < TOL, "Q=0 LSE = ln Nk"
    o, lse = attn(q, k, v, 0.25, True)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.abs(o - prefix_mean).max() < TOL, "Q=0 causal prefix mean"
    assert np.abs(lse - np.log(np.arange(1, n + 1))).max() < TOL, "Q=0 causal LSE = ln(i+1)"


def check_single_key(attn):
    """Nk = 1 => O = v_0 and LSE = scale * q . k_0; causal row 0 => O_0 = v_0."""
    q, k, v = _rand_head(8, 5, 1, 6)
    o, lse = attn(q, k, v, 0.37, False)
    assert np.abs(o - v[0]).max() < TOL, "Nk=1 O"
    assert np.abs(lse - 0.37 * (q @ k[0])).max() < TOL, "Nk=1 LSE"
    q, k, v = _rand_head(9, 6, 6, 3)
    o, lse = attn(q, k, v, 0.37, True)
    assert np.abs(o[0] - v[0]).max() < TOL, "causal row 0 attends only key 0"
    assert abs(lse[0] - 0.37 * (q[0] @ k[0])) < TOL, "causal row 0 LSE"


def check_causal_prefix(attn):
    """Causal row i equals non-causal attention of q_i over keys/values 0..i."""
    n = 9
    q, k, v = _rand_head(10, n, n, 5)
    oc, lc = attn(q, k, v, 0.45, True)
    for i in range(n):
        o1, l1 = attn(q[i:i + 1], k[:i + 1], v[:i + 1], 0.45, False)
        assert np.abs(oc[i] - o1[0]).max() < TOL and abs(lc[i] - l1[0]) < TOL, f"causal prefix row {i}"


def check_shift(attn):
    """K_j += u for every j  =>  O unchanged, LSE_i += scale * q_i . u (Day-21 §5.2 invariance)."""
    q, k, v = _rand_head(11, 8, 14, 4)
    u = _rng(12).standard_normal(4)
    o1, l1 = attn(q, k, v, 0.6, False)
    o2, l2 = attn(q, k + u, v, 0.6, False)
    assert np.abs(o1 - o2).max() < 1e-10, "shift O"
    assert np.abs(l2 - (l1 + 0.6 * (q @ u))).max() < 1e-10, "shift LSE"


def check_overflow(attn):
    """Scores around +-1000 (exp would overflow without the max subtraction): finite results,
    LSE within [max score, max score + ln Nk]."""
    q, k, v = _rand_head(13, 6, 20, 3)
    k = k * 400.0
    o, lse = attn(q, k, v, 1.0, False)
    s = q @ k.T
    assert np.isfinite(o).all() and np.isfinite(lse).all(), "overflow: finite"
    assert (lse >= s.max(axis=1) - 1e-9).all() and (lse <= s.max(axis=1) + math.log(20) + 1e-9).all()
    assert np.abs(o).max() <= np.abs(v).max() + 1e-12, "O is a convex combination of V rows"


def check_scipy(attn):
    """Rows of softmax / logsumexp agree with scipy.special (library special case)."""
    from scipy.special import softmax, logsumexp
    n, d = 11, 6
    q, k, _ = _rand_head(14, n, n, d)
    for causal in (False, True):
        p, lse = attn(q, k, np.eye(n), 0.8, causal)
        s = 0.8 * (q @ k.T)
        if causal:
            s = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, s)
        assert np.abs(p - softmax(s, axis=1)).max() < TOL, "scipy softmax"
        assert np.abs(lse - logsumexp(s, axis=1)).max() < TOL, "scipy logsumexp"


def check_torch_sdpa(attn):
    """O agrees with torch's scaled_dot_product_attention on CPU in float64 (independent code)."""
    import torch
    for nq, nk, d, causal in [(13, 29, 8, False), (17, 17, 16, True), (1, 40, 4, False)]:
        q, k, v = _rand_head(15 + nq, nq, nk, d)
        o, _ = attn(q, k, v, 1.0 / math.sqrt(d), causal)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            is_causal=causal, scale=1.0 / math.sqrt(d))[0].numpy()
        assert np.abs(o - ref).max() < 1e-12, "torch SDPA"


ALL_CHECKS = [
    check_brute_force, check_constant_v, check_one_hot_rowsum, check_permutation_invariance,
    check_zero_query, check_single_key, check_causal_prefix, check_shift, check_overflow,
    check_scipy, check_torch_sdpa,
]


def failures(attn):
    """Names of the checks that `attn` violates (exceptions count as violations)."""
    bad = []
    for chk in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                chk(attn)
        except Exception:  # noqa: BLE001 - any failure, including NaN-driven errors, counts
            bad.append(chk.__name__)
    return bad
