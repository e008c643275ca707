"""Element masks for the masked forward: seeded generators and the bit-packed storage form.

No attention arithmetic here.  A mask is a boolean matrix allowed [Nq, Nk] (key j visible to
query row i iff allowed[i, j]); the library takes it bit-packed, one 64-bit word per query row per
64 keys: bit (j % 64) of word [i][j // 64] is allowed[i, j], and bits of keys past Nk are 0.

Generators:
  * documents(N, seed, min_len, max_len): N tokens packed from documents of seeded random
    lengths, each token attending causally within its own document (the mask of packed
    training sequences: off-diagonal blocks empty, blocks inside a document full, document
    boundaries and the diagonal partial);
  * sliding_window(Nq, Nk, window): causal, and only the last `window` keys;
  * random_tiles(Nq, Nk, seed, bq, bk, ...): tiles of bq x bk elements that are empty, full or
    random bit by bit, at a granularity of the caller's choosing (so that tile edges need not
    line up with any kernel tiling).
"""
from __future__ import annotations

import numpy as np


def documents(n: int, seed: int, min_len: int, max_len: int) -> np.ndarray:
    g = np.random.default_rng(seed)
    doc = np.empty(n, dtype=np.int64)
    start, d = 0, 0
    while start < n:
        length = int(g.integers(min_len, max_len + 1))
        doc[start:start + length] = d
        start += length
        d += 1
    i = np.arange(n)
    return (doc[:, None] == doc[None, :]) & (i[None, :] <= i[:, None])


def sliding_window(nq: int, nk: int, window: int) -> np.ndarray:
    i = np.arange(nq)[:, None] + (nk - nq)  # bottom-right aligned: the last query sees the last key
    j = np.arange(nk)[None, :]
    return (j <= i) & (j > i - window)


def random_tiles(nq: int, nk: int, seed: int, bq: int, bk: int, p_empty: float = 0.4, p_full: float = 0.3,
                 p_bit: float = 0.5, empty_rows: tuple = ()) -> np.ndarray:
    g = np.random.default_rng(seed)
    tq, tk = -(-nq // bq), -(-nk // bk)
    cls = g.choice(3, size=(tq, tk), p=[p_empty, p_full, 1.0 - p_empty - p_full])
    bits = g.random((nq, nk)) < p_bit
    big = np.repeat(np.repeat(cls, bq, axis=0), bk, axis=1)[:nq, :nk]
    m = np.where(big == 1, True, np.where(big == 0, False, bits))
    for r in empty_rows:
        m[r] = False
    return m


def pack_bits(allowed: np.ndarray) -> np.ndarray:
    """[Nq, Nk] booleans -> [Nq, ceil(Nk / 64)] uint64 words (bit j % 64 of word j // 64)."""
    a = np.asarray(allowed, dtype=bool)
    nq, nk = a.shape
    nt = -(-nk // 64)
    padded = np.zeros((nq, nt * 64), dtype=bool)
    padded[:, :nk] = a
    by = np.packbits(padded.reshape(nq, nt, 8, 8), axis=-1, bitorder="little")[..., 0]  # [nq, nt, 8] bytes
    return np.ascontiguousarray(by).view(np.uint64).reshape(nq, nt)


def unpack_bits(words: np.ndarray, nk: int) -> np.ndarray:
    w = np.ascontiguousarray(words, dtype=np.uint64)
    nq, nt = w.shape
    by = w.view(np.uint8).reshape(nq, nt, 8)
    return np.unpackbits(by, axis=-1, bitorder="little").reshape(nq, nt * 64)[:, :nk].astype(bool)


def element_mask(w) -> np.ndarray:
    """The boolean [Nq, Nk] mask of a workload's mask_rule."""
    rule = w.mask_rule
    if rule[0] == "documents":
        if w.Nq != w.Nk:
            raise ValueError("the document mask needs Nq == Nk")
        return documents(w.Nq, rule[1], rule[2], rule[3])
    if rule[0] == "window":
        return sliding_window(w.Nq, w.Nk, rule[1])
    if rule[0] == "tiles":
        return random_tiles(w.Nq, w.Nk, rule[1], rule[2], rule[3], *rule[4:])
    raise ValueError(f"unknown mask rule {rule!r}")


def visible_pairs(allowed: np.ndarray) -> int:
    return int(np.count_nonzero(allowed))
