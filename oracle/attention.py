"""Exact attention, written as its plain definition, in float64 (test infrastructure only).

What is computed (Day-21 page §3.1 "standard implementation data flow" and §5.1;
M4-047 card §3):
    S   = scale * Q K^T                       (Nq x Nk; scale = 1/sqrt(d) in the pages)
    S_ij = -inf where j > i + diag            (causal mask, only when requested; diag = 0 is
                                               the usual top-left diagonal, diag = Nk - Nq puts
                                               the last query on the last key: a chunk of new
                                               queries appended to a KV cache)
    m_i = max_j S_ij                          (pass 1 of the safe softmax, Day-21 §5.1)
    e_ij = exp(S_ij - m_i), l_i = sum_j e_ij  (pass 2)
    P   = e / l,  O = P V
    LSE_i = m_i + ln(l_i)                     (the per-row statistic kept for the backward
                                               recompute, M4-047 card §3 point (c))

Rows may be processed in chunks to bound memory, but every chunk spans all keys,
so each row's two passes see the whole row.  Nothing here uses the online recurrence.

Arbitrary masks (the "skip masked blocks, mask partial ones element by element" rule of the
Day-21 page's §6 table, and the arbitrary masks FlashAttention-2 is said to lack in the Q31
answer §2): an element mask `allowed` [Nq, Nk] of booleans, key j visible to query row i iff
allowed[i, j]; S_ij = -inf where it is not.  A row with no visible key has an empty softmax:
its O row is 0 (a sum over no keys) and its LSE is ln 0 = -inf.

Grouped K/V heads (GQA: several query heads share one K/V head; the Day-21 page's FAQ Q5 lists
it among the techniques that matter at decode, where reading the KV cache is the bottleneck):
with H query heads and H_kv K/V heads, H_kv dividing H, query head h reads K/V head
h // (H / H_kv).  H_kv = H is ordinary multi-head attention.

Split-KV decode (Q31 answer, follow-up 3: split K/V into chunks processed in parallel,
then merge; the merge rescales with exp(m_block - m_global), follow-up 2):
    split_partials  per split s over keys [a_s, b_s): m_s, l_s = sum exp(S - m_s),
                    O_s = sum_j exp(S_j - m_s) v_j (unnormalised)
    combine_partials M = max_s m_s, w_s = exp(m_s - M), L = sum w_s l_s,
                    O = sum w_s O_s / L, LSE = M + ln L; an empty split (m_s = -inf,
                    l_s = 0) has weight 0.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def scores(q, k, scale: float) -> np.ndarray:
    """S = scale * q k^T of one head (no mask)."""
    return float(scale) * (_f64(q) @ _f64(k).T)


def softmax_two_pass(s: np.ndarray):
    """Row-wise safe softmax in two passes: returns (P, m, l)."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    return e / l, m[..., 0], l[..., 0]


def attention_head(q, k, v, scale: float, causal: bool = False, rows=None, row_chunk: int = 1024,
                   diag: int = 0, allowed=None):
    """One head. q [Nq, d], k and v [Nk, d] -> (O [n, d], LSE [n]) in float64.

    rows: optional increasing 1-D array of query row indices to compute (the masks use the
    true row index); default all rows.  causal: key j is visible to query row i iff
    j <= i + diag.  allowed: optional boolean element mask [Nq, Nk] (key j visible to row i iff
    allowed[i, j]); a row it leaves without keys gets O = 0 and LSE = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    o = np.empty((len(rows), v.shape[1]), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    for c0 in range(0, len(rows), row_chunk):
        r = rows[c0:c0 + row_chunk]
        s = float(scale) * (q[r] @ k.T)
        if causal:
            s = np.where(np.arange(k.shape[0])[None, :] > r[:, None] + diag, -np.inf, s)
        if allowed is not None:
            s = np.where(np.asarray(allowed, dtype=bool)[r], s, -np.inf)
            empty = np.isneginf(s).all(axis=1)
            s[empty] = 0.0  # placeholder scores for rows without keys; their results are set below
        p, m, l = softmax_two_pass(s)
        o[c0:c0 + len(r)] = p @ v
        lse[c0:c0 + len(r)] = m + np.log(l)
        if allowed is not None:
            o[c0:c0 + len(r)][empty] = 0.0
            lse[c0:c0 + len(r)][empty] = -np.inf
    return o, lse


def attention(q, k, v, scale: float, causal: bool = False, row_chunk: int = 1024, diag: int = 0, allowed=None):
    """[B, H, Nq, d] x [B, H_kv, Nk, d] x [B, H_kv, Nk, d] -> (O [B, H, Nq, d], LSE [B, H, Nq]) float64.

    H_kv must divide H; query head h attends with K/V head h // (H // H_kv).  allowed: one
    element mask [Nq, Nk] for every batch and head (see attention_head)."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    B, H, Nq, _ = q.shape
    H_kv = k.shape[1]
    if H % H_kv != 0 or v.shape[1] != H_kv:
        raise ValueError(f"H_kv = {H_kv} K/V heads do not divide H = {H} query heads")
    group = H // H_kv
    o = np.empty(q.shape[:3] + (v.shape[-1],), dtype=np.float64)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, h // group], v[b, h // group], scale, causal,
                                                row_chunk=row_chunk, diag=diag, allowed=allowed)
    return o, lse


def attention_probs(q, k, scale: float) -> np.ndarray:
    """The full probability matrix P of one head, no mask (small inputs only)."""
    p, _, _ = softmax_two_pass(scores(q, k, scale))
    return p


def split_bounds(nk: int, num_splits: int):
    """Contiguous splits of ceil(nk / num_splits) keys; trailing splits may be short or empty."""
    chunk = -(-nk // num_splits)
    return [(min(nk, s * chunk), min(nk, (s + 1) * chunk)) for s in range(num_splits)]


def split_partials(q, k, v, scale: float, num_splits: int):
    """One query q [d] against k, v [Nk, d]: per-split (O_s [S, d], m_s [S], l_s [S])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S = num_splits
    o = np.zeros((S, v.shape[1]), dtype=np.float64)
    m = np.full(S, -np.inf, dtype=np.float64)
    l = np.zeros(S, dtype=np.float64)
    for s, (a, b) in enumerate(split_bounds(k.shape[0], S)):
        if b <= a:
            continue  # empty split: m = -inf, l = 0, O = 0
        x = float(scale) * (k[a:b] @ q)
        m[s] = x.max()
        e = np.exp(x - m[s])
        l[s] = e.sum()
        o[s] = e @ v[a:b]
    return o, m, l


def combine_partials(o_s, m_s, l_s):
    """Merge split partials: (O [d], LSE) in float64."""
    o_s, m_s, l_s = _f64(o_s), _f64(m_s), _f64(l_s)
    M = m_s.max()
    w = np.where(np.isneginf(m_s), 0.0, np.exp(m_s - M))
    L = float((w * l_s).sum())
    return (w @ o_s) / L, M + math.log(L)
