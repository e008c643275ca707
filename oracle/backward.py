"""Gradients of exact attention, written as their plain definition, in float64 (test
infrastructure only).

The backward pass the M4-047 card ("高效注意力与 FlashAttention", §3 point (c)) refers to: the
forward keeps only O and the per-row statistic, and the backward recomputes what it needs
instead of storing the N x N probabilities (which the Day-21 page, §3.2, notes a standard
implementation has to keep for training).  The pages do not write the gradients out; they are
the chain rule through the definition in attention.py.  For one head, with a loss whose
gradient with respect to O is dO:

    P   = softmax(S),  S = scale * Q K^T (masked entries -inf, so P = 0 there)
    dV  = P^T dO                              (O = P V)
    dP  = dO V^T
    dS  = P * (dP - rowsum(P * dP))           (softmax Jacobian, row by row)
    dQ  = scale * dS K,   dK = scale * dS^T Q

rowsum(P * dP)_i equals dO_i . O_i, the form a recomputing kernel uses.  Here P comes from the
two-pass definition, not from a saved statistic.  With grouped K/V heads the gradient of a K/V
head is the sum over the query heads that read it.
"""
from __future__ import annotations

import numpy as np

from .attention import softmax_two_pass


def attention_backward_head(q, k, v, do, scale: float, causal: bool = False, diag: int = 0):
    """One head: q [Nq, d], k and v [Nk, d], do [Nq, d] -> (dq, dk, dv) in float64."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = float(scale) * (q @ k.T)
    if causal:
        i = np.arange(s.shape[0])[:, None]
        j = np.arange(s.shape[1])[None, :]
        s = np.where(j > i + diag, -np.inf, s)
    p, _, _ = softmax_two_pass(s)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, do, scale: float, causal: bool = False, diag: int = 0):
    """[B, H, Nq, d] q and do, [B, H_kv, Nk, d] k and v -> (dq [B,H,Nq,d], dk, dv [B,H_kv,Nk,d]).

    H_kv must divide H; query head h reads K/V head h // (H // H_kv), whose gradients sum over
    those query heads."""
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    B, H = q.shape[:2]
    H_kv = k.shape[1]
    if H % H_kv != 0 or v.shape[1] != H_kv:
        raise ValueError(f"H_kv = {H_kv} K/V heads do not divide H = {H} query heads")
    group = H // H_kv
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            a, bk, bv = attention_backward_head(q[b, h], k[b, h // group], v[b, h // group], do[b, h], scale,
                                                causal, diag)
            dq[b, h] = a
            dk[b, h // group] += bk
            dv[b, h // group] += bv
    return dq, dk, dv


def softmax_row_stat(o, do) -> np.ndarray:
    """rowsum(dO * O) over the last axis: the per-row term a recomputing backward subtracts."""
    return (np.asarray(o, dtype=np.float64) * np.asarray(do, dtype=np.float64)).sum(axis=-1)


__all__ = ["attention_backward_head", "attention_backward", "softmax_row_stat"]
