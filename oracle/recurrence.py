"""The online-softmax block recurrence, in pure Python (test infrastructure only; tiny inputs).

It exists to pin the block-by-block steps that the GPU kernels perform against the
two-pass definition in attention.py.  Written from the Day-21 page:
  §5.2: keep a running maximum m and a running, rescaled sum l; when a block with
        maximum m_blk arrives, m_new = max(m_old, m_blk) and
        l_new = exp(m_old - m_new) * l_old + sum_blk exp(x - m_new);
  §5.3: for attention also keep an accumulator O_acc, rescaled by the same factor
        before the block's exp(S_blk - m_new) V_blk is added; divide by l only at the end.
and from the Q31 answer, follow-up 2: merging two partial results rescales the one with
the smaller maximum by exp(m_small - m_large) (its example: maxima 10 and 12, factor exp(-2)).

The initial state is m = -inf, l = 0, so the first block's rescale factor is exp(-inf) = 0.

A plain softmax of a vector x is the special case of one query q = [1], keys [x_j] (d = 1),
scale 1 and one-hot value rows: the output row is then softmax(x) itself.
"""
from __future__ import annotations

import math


def _exp(x: float) -> float:
    return 0.0 if x == -math.inf else math.exp(x)


def attention_row(q, keys, values, scale: float, block: int):
    """One query row against lists of key and value rows, block by block (Day-21 §5.3).

    Returns (o: list[float], lse: float).  Keys that are masked out are simply not passed.
    """
    d = len(values[0])
    m, l = -math.inf, 0.0
    acc = [0.0] * d
    for j0 in range(0, len(keys), block):
        s = [scale * sum(a * b for a, b in zip(q, kj)) for kj in keys[j0:j0 + block]]
        m_new = max(m, max(s))
        alpha = _exp(m - m_new)
        p = [math.exp(t - m_new) for t in s]
        l = alpha * l + sum(p)
        acc = [alpha * a for a in acc]
        for pj, vj in zip(p, values[j0:j0 + block]):
            acc = [a + pj * b for a, b in zip(acc, vj)]
        m = m_new
    return [a / l for a in acc], m + math.log(l)


def partial_state(q, keys, values, scale: float):
    """(m, l, acc) of one chunk of keys: the unnormalised state a split-KV worker produces."""
    if not keys:
        return -math.inf, 0.0, [0.0] * len(q)
    s = [scale * sum(a * b for a, b in zip(q, kj)) for kj in keys]
    m = max(s)
    p = [math.exp(t - m) for t in s]
    acc = [0.0] * len(values[0])
    for pj, vj in zip(p, values):
        acc = [a + pj * b for a, b in zip(acc, vj)]
    return m, sum(p), acc


def merge_states(a, b):
    """Merge two (m, l, acc) states (Q31 answer follow-up 2): rescale each by exp(m_i - max)."""
    (ma, la, acca), (mb, lb, accb) = a, b
    m = max(ma, mb)
    if m == -math.inf:
        return a
    fa, fb = _exp(ma - m), _exp(mb - m)
    return m, fa * la + fb * lb, [fa * x + fb * y for x, y in zip(acca, accb)]


def finish(state):
    """(m, l, acc) -> (o, lse)."""
    m, l, acc = state
    return [a / l for a in acc], m + math.log(l)
