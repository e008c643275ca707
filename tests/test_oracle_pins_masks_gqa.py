"""Pins of the float64 reference for the two generalisations the library's extended entry points
take (CPU only):

  * the causal mask with a diagonal offset: key j visible to query i iff j <= i + diag, with
    diag = 0 (top-left, the usual causal mask, any Nq and Nk) or diag = Nk - Nq (bottom-right:
    a chunk of Nq new queries appended to a cache of Nk keys, the last query seeing every key);
  * grouped K/V heads: query head h of H reads K/V head h // (H / H_kv).

They are checked against a pure-Python brute-force evaluation of the textbook softmax with the
offset mask, against torch's scaled_dot_product_attention on the CPU in float64 (an explicit
boolean mask, and its own grouped-head mode), and against relations the definitions force (a
bottom-right chunk equals the last rows of the full causal problem; a one-query chunk sees every
key; grouping equals repeating each K/V head).  Broken copies of the reference show that each
plausible mistake in the offset or in the head mapping is caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def brute_force_offset(q, k, v, scale, diag):
    """Textbook softmax (no max subtraction, exact sums) with mask j > i + diag; pure Python."""
    nq, nk, dv = len(q), len(k), len(v[0])
    o = np.zeros((nq, dv))
    lse = np.zeros(nq)
    for i in range(nq):
        allowed = [j for j in range(nk) if j <= i + diag]
        e = {j: math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j]))) for j in allowed}
        den = math.fsum(e.values())
        for c in range(dv):
            o[i, c] = math.fsum(e[j] * float(v[j][c]) for j in allowed) / den
        lse[i] = math.log(den)
    return o, lse


SHAPES = [(1, 1), (3, 5), (5, 3), (4, 9), (7, 7), (1, 6), (6, 1), (9, 4)]


def _offsets(nq, nk):
    out = [0]  # top-left: every row sees key 0
    if nk >= nq:
        out.append(nk - nq)  # bottom-right
    return out


# ------------------------------------------------------------- checks on a one-head function
def check_brute_force(attn):
    for seed, (nq, nk) in enumerate(SHAPES):
        g = _rng(300 + seed)
        d = 3
        q, k, v = g.standard_normal((nq, d)), g.standard_normal((nk, d)), g.standard_normal((nk, d))
        for diag in _offsets(nq, nk):
            o, lse = attn(q, k, v, 0.7, True, diag)
            ob, lb = brute_force_offset(q.tolist(), k.tolist(), v.tolist(), 0.7, diag)
            assert np.abs(o - ob).max() < TOL, f"brute force O ({nq}, {nk}, diag {diag})"
            assert np.abs(lse - lb).max() < TOL, f"brute force LSE ({nq}, {nk}, diag {diag})"


def check_torch_masked(attn):
    """torch SDPA with an explicit boolean mask tril(diagonal=diag) (True = may attend)."""
    for seed, (nq, nk) in enumerate([(16, 40), (40, 16), (33, 33), (8, 100)]):
        g = _rng(400 + seed)
        d = 8
        q, k, v = g.standard_normal((nq, d)), g.standard_normal((nk, d)), g.standard_normal((nk, d))
        for diag in _offsets(nq, nk):
            mask = torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=diag)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None], torch.from_numpy(v)[None, None],
                attn_mask=mask, scale=0.3)[0, 0].numpy()
            o, _ = attn(q, k, v, 0.3, True, diag)
            assert np.abs(o - ref).max() < 1e-10, f"torch SDPA ({nq}, {nk}, diag {diag})"


def check_chunk_is_tail_of_full_causal(attn):
    """Bottom-right on the last Nq queries == those rows of the full top-left causal problem."""
    g = _rng(5)
    nk, d = 48, 6
    qf, k, v = g.standard_normal((nk, d)), g.standard_normal((nk, d)), g.standard_normal((nk, d))
    of, lf = attn(qf, k, v, 0.4, True, 0)
    for nq in (1, 5, 17, 48):
        oc, lc = attn(qf[nk - nq:], k, v, 0.4, True, nk - nq)
        assert np.abs(oc - of[nk - nq:]).max() < TOL and np.abs(lc - lf[nk - nq:]).max() < TOL, f"chunk {nq}"


def check_single_query_sees_everything(attn):
    g = _rng(6)
    q, k, v = g.standard_normal((1, 5)), g.standard_normal((30, 5)), g.standard_normal((30, 5))
    o1, l1 = attn(q, k, v, 0.5, True, 29)
    o0, l0 = attn(q, k, v, 0.5, False, 0)
    assert np.abs(o1 - o0).max() < TOL and np.abs(l1 - l0).max() < TOL


def check_offset_row_closed_form(attn):
    """Q = 0: row i is the mean of the visible V rows and LSE_i = ln(#visible)."""
    g = _rng(7)
    nq, nk, d = 6, 11, 4
    q, k, v = np.zeros((nq, d)), g.standard_normal((nk, d)), g.standard_normal((nk, d))
    for diag in (0, nk - nq):
        o, lse = attn(q, k, v, 1.0, True, diag)
        for i in range(nq):
            n = min(nk, i + diag + 1)
            assert abs(lse[i] - math.log(n)) < TOL
            assert np.abs(o[i] - v[:n].mean(axis=0)).max() < TOL


HEAD_CHECKS = [check_brute_force, check_torch_masked, check_chunk_is_tail_of_full_causal,
               check_single_query_sees_everything, check_offset_row_closed_form]


def head_failures(attn):
    out = []
    for c in HEAD_CHECKS:
        try:
            c(attn)
        except AssertionError as e:
            out.append(f"{c.__name__}: {e}")
    return out


# ------------------------------------------------------------- checks on a batched function
def check_gqa_torch(attn_b):
    """torch SDPA's own grouped-head mode (enable_gqa) on the CPU in float64."""
    g = _rng(8)
    B, H, Hkv, nq, nk, d = 2, 8, 2, 9, 13, 4
    q = g.standard_normal((B, H, nq, d))
    k, v = g.standard_normal((B, Hkv, nk, d)), g.standard_normal((B, Hkv, nk, d))
    for causal, diag in ((False, 0), (True, 0), (True, nk - nq)):
        mask = torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=diag) if causal else None
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=0.5,
            enable_gqa=True).numpy()
        o, _ = attn_b(q, k, v, 0.5, causal, diag)
        assert np.abs(o - ref).max() < 1e-10, f"torch enable_gqa (causal {causal}, diag {diag})"


def check_gqa_equals_repeated_heads(attn_b):
    g = _rng(9)
    B, H, nq, nk, d = 1, 6, 5, 7, 3
    q = g.standard_normal((B, H, nq, d))
    for Hkv in (1, 2, 3, 6):
        k, v = g.standard_normal((B, Hkv, nk, d)), g.standard_normal((B, Hkv, nk, d))
        rep = H // Hkv
        o, l = attn_b(q, k, v, 0.6, True, nk - nq)
        o1, l1 = attn_b(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), 0.6, True, nk - nq)
        assert np.abs(o - o1).max() < TOL and np.abs(l - l1).max() < TOL, f"H_kv {Hkv}"
        for h in range(H):  # and each head against the brute force with its own K/V head
            ob, lb = brute_force_offset(q[0, h].tolist(), k[0, h // rep].tolist(), v[0, h // rep].tolist(), 0.6,
                                        nk - nq)
            assert np.abs(o[0, h] - ob).max() < TOL and np.abs(l[0, h] - lb).max() < TOL, f"head {h}"


BATCH_CHECKS = [check_gqa_torch, check_gqa_equals_repeated_heads]


def batch_failures(attn_b):
    out = []
    for c in BATCH_CHECKS:
        try:
            c(attn_b)
        except AssertionError as e:
            out.append(f"{c.__name__}: {e}")
    return out


# ------------------------------------------------------------- the reference and broken copies
def ref_head(q, k, v, scale, causal, diag):
    return oracle.attention_head(q, k, v, scale, causal, diag=diag)


def ref_batched(q, k, v, scale, causal, diag):
    return oracle.attention(q, k, v, scale, causal, diag=diag)


def test_reference_passes_offset_checks():
    assert head_failures(ref_head) == []


def test_reference_passes_grouped_head_checks():
    assert batch_failures(ref_batched) == []


def test_reference_rejects_non_dividing_kv_heads():
    x = np.zeros((1, 6, 2, 2))
    with pytest.raises(ValueError):
        oracle.attention(x, np.zeros((1, 4, 2, 2)), np.zeros((1, 4, 2, 2)), 1.0)


def _broken_head(q, k, v, scale, causal, diag, *, mistake):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    s = scale * (q @ k.T)
    i = np.arange(s.shape[0])[:, None]
    j = np.arange(s.shape[1])[None, :]
    if causal:
        masked = {"offset_sign": j > i - diag, "offset_ignored": j > i, "offset_strict": j >= i + diag,
                  "offset_on_keys": j + diag > i}.get(mistake, j > i + diag)
        s = np.where(masked, -np.inf, s)
    with np.errstate(invalid="ignore", divide="ignore"):  # a broken mask can hide whole rows
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        return (e / l) @ v, (m + np.log(l)).reshape(-1)


def _broken_batched(q, k, v, scale, causal, diag, *, mistake):
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    o = np.empty(q.shape[:3] + (v.shape[-1],))
    lse = np.empty(q.shape[:3])
    for b in range(B):
        for h in range(H):
            kh = {"kv_modulo": h % Hkv, "kv_times": min(Hkv - 1, h * Hkv // H + (1 if h % 2 else 0))}.get(
                mistake, h // (H // Hkv))
            o[b, h], lse[b, h] = oracle.attention_head(q[b, h], k[b, kh], v[b, kh], scale, causal, diag=diag)
    return o, lse


@pytest.mark.parametrize("mistake", ["offset_sign", "offset_ignored", "offset_strict", "offset_on_keys"])
def test_planted_offset_mistake_is_caught(mistake):
    assert head_failures(lambda *a: _broken_head(*a, mistake=mistake)), f"{mistake} slipped through"


def test_unbroken_offset_copy_passes():
    assert head_failures(lambda *a: _broken_head(*a, mistake=None)) == []


@pytest.mark.parametrize("mistake", ["kv_modulo", "kv_times"])
def test_planted_head_mapping_mistake_is_caught(mistake):
    assert batch_failures(lambda *a: _broken_batched(*a, mistake=mistake)), f"{mistake} slipped through"


def test_unbroken_head_mapping_copy_passes():
    assert batch_failures(lambda *a: _broken_batched(*a, mistake=None)) == []
