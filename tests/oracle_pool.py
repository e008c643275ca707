"""Whole-workload parity: the float64 reference computed head by head in worker processes.

Comparing every head of a full-size workload needs the reference on every head, about one
second of one host core per 8192 x 8192 head.  The work is spread over a pool of worker
processes.  The pool is forked once, when the tests that use it have been collected and before
any test runs, so it is forked from a process that has not initialised the GPU runtime (such a
process must not fork).  The workers never touch the GPU: each regenerates its head's inputs
from the seeded recipe (synth) and runs the reference with one BLAS thread.

Test infrastructure only, like the reference itself.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time

import numpy as np

_POOL = None


def _init_worker():
    import threadpoolctl
    threadpoolctl.threadpool_limits(1)


def start():
    """Fork the pool (idempotent).  Call only before the GPU runtime is initialised."""
    global _POOL
    if _POOL is None:
        _POOL = mp.get_context("fork").Pool(min(16, len(os.sched_getaffinity(0))), initializer=_init_worker)
    return _POOL


def stop():
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL = None


def pool():
    if _POOL is None:
        raise RuntimeError("the reference pool was not forked at collection time")
    return _POOL


_MASK = {}


def _allowed(w):
    """The workload's element mask (None without one), built once per worker."""
    if not w.mask_rule:
        return None
    key = (w.Nq, w.Nk, w.mask_rule)
    if key not in _MASK:
        from synth import masks
        _MASK.clear()
        _MASK[key] = masks.element_mask(w)
    return _MASK[key]


def _head_job(args):
    """(w, b, h) -> (b, h, O [Nq, d], LSE [Nq]) float64 from the reference on regenerated inputs."""
    import oracle
    from synth import inputs as si
    w, b, h = args
    hk = h // (w.H // w.kv_heads)
    q = si.head_block_f32(w, "q", b, h)
    k = si.head_block_f32(w, "k", b, hk)
    v = si.head_block_f32(w, "v", b, hk)
    o, lse = oracle.attention_head(q, k, v, w.scale, w.causal, diag=w.diag, allowed=_allowed(w))
    return b, h, o, lse


def edge_rows(n: int) -> np.ndarray:
    """The first and last rows and those around 32/64/128/256-row boundaries and the middle."""
    e = {0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 129, 255, 256, 257, n // 2, n - 257, n - 256, n - 129, n - 128,
         n - 65, n - 64, n - 33, n - 32, n - 2, n - 1}
    return np.array(sorted(r for r in e if 0 <= r < n))


class _Acc:
    """Whole-tensor error statistics accumulated head by head."""

    def __init__(self):
        self.ss_diff = self.ss_ref = 0.0
        self.o_maxabs = self.lse_maxabs = self.lse_maxrel = self.worst_row = 0.0
        self.finite = True
        self.n = 0

    def add(self, o, lse, o_ref, lse_ref):
        o, lse = np.asarray(o, np.float64), np.asarray(lse, np.float64)
        d = o - o_ref
        self.ss_diff += float((d * d).sum())
        self.ss_ref += float((o_ref * o_ref).sum())
        self.o_maxabs = max(self.o_maxabs, float(np.abs(d).max()))
        self.worst_row = max(self.worst_row, float(np.sqrt((d.reshape(-1, d.shape[-1]) ** 2).sum(-1)).max()))
        dl = np.abs(lse - lse_ref)
        self.lse_maxabs = max(self.lse_maxabs, float(dl.max()))
        self.lse_maxrel = max(self.lse_maxrel, float((dl / np.maximum(np.abs(lse_ref), 1e-30)).max()))
        self.finite &= bool(np.isfinite(o).all() and np.isfinite(lse).all())
        self.n += 1

    def metrics(self) -> dict:
        return {"o_maxabs": self.o_maxabs, "o_rel_l2": float(np.sqrt(self.ss_diff / self.ss_ref)),
                "o_worst_row_l2": self.worst_row, "lse_maxabs": self.lse_maxabs, "lse_maxrel": self.lse_maxrel,
                "finite": self.finite, "heads": self.n}


def compare_every_head(w, o_gpu: np.ndarray, lse_gpu: np.ndarray):
    """The GPU's o [B,H,Nq,d] and lse [B,H,Nq] (host float32) against the reference on every head.

    Returns (metrics over the whole tensor, metrics over the edge rows of every head, the worst
    head by O's max-abs error as (b, h, max-abs))."""
    jobs = [(w, b, h) for b in range(w.B) for h in range(w.H)]
    whole, edges = _Acc(), _Acc()
    er = edge_rows(w.Nq)
    worst = (None, None, -1.0)
    t0 = last = time.perf_counter()
    for b, h, o_ref, l_ref in pool().imap_unordered(_head_job, jobs, chunksize=1):
        if time.perf_counter() - last > 10.0:
            last = time.perf_counter()
            print(f"    reference: {whole.n} of {len(jobs)} heads compared, {last - t0:.0f} s", flush=True)
        og, lg = o_gpu[b, h], lse_gpu[b, h]
        whole.add(og, lg, o_ref, l_ref)
        edges.add(og[er], lg[er], o_ref[er], l_ref[er])
        e = float(np.abs(og.astype(np.float64) - o_ref).max())
        if e > worst[2]:
            worst = (b, h, e)
    return whole.metrics(), edges.metrics(), worst
