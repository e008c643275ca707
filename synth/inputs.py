"""Seeded synthetic inputs.

Recipe (every workload):
  * each (tensor, batch, head) block of shape [rows, d] is drawn independently as
    float32 N(0, 1) from numpy's PCG64 seeded with SeedSequence([seed, tensor_id, b, h]),
    tensor_id 0 = Q, 1 = K, 2 = V, 3 = dO (the output gradient a backward test feeds in);
  * K is then multiplied by the workload's power-of-two factors (exact in bf16);
  * bf16 workloads round the float32 draw to bf16 with round-to-nearest-even.

The canonical input is the stored bit pattern (uint16 for bf16, float32 for f32):
the GPU library and the reference implementation consume exactly the same values.
Per-head seeding lets a test regenerate one head's inputs on the host without
materialising the whole tensor.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .workloads import Workload

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}  # "do": the gradient fed to the backward


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Inputs here are finite normals, so no NaN handling is needed; a value whose
    rounding carries into the exponent field rounds up correctly by construction.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact widening)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(seed: int, tensor_id: int, b: int, h: int, rows: int, d: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, b, h])))
    return g.standard_normal((rows, d), dtype=np.float32)


def _apply_k_rule(x: np.ndarray, rule: tuple) -> np.ndarray:
    kind = rule[0]
    if kind == "none":
        return x
    if kind == "scale_all":
        return x * np.float32(rule[1])
    if kind == "scale_rows_every":
        every, factor = rule[1], np.float32(rule[2])
        x = x.copy()
        x[::every] *= factor
        return x
    raise ValueError(f"unknown K rule {rule!r}")


def head_block(w: Workload, which: str, b: int, h: int) -> np.ndarray:
    """One (b, h) block of Q, K or V in storage form ([rows, d] uint16 bf16 bits or float32)."""
    rows = w.Nq if which in ("q", "do") else w.Nk
    x = _draw(w.seed, TENSOR_IDS[which], b, h, rows, w.d)
    if which == "k":
        x = _apply_k_rule(x, w.k_rule)
    if w.dtype == "bf16":
        return round_to_bf16_bits(x)
    return x


E4M3_MAX = 448.0  # largest finite OCP FP8 E4M3 value


def head_block_fp8(w: Workload, which: str, b: int, h: int):
    """One (b, h) block of Q, K or V as OCP FP8 E4M3 codes ([rows, d] uint8) and its scale: the
    float32 draw x (with the K rule) is stored as codes of x / scale, scale = max|x| / 448, rounded
    to nearest even by torch's float8_e4m3fn conversion.  Input preparation only: the values a
    kernel and the reference see are the codes and the scale."""
    import torch

    rows = w.Nq if which in ("q", "do") else w.Nk
    x = _draw(w.seed, TENSOR_IDS[which], b, h, rows, w.d)
    if which == "k":
        x = _apply_k_rule(x, w.k_rule)
    amax = float(np.abs(x).max())
    scale = np.float32(amax / E4M3_MAX if amax > 0 else 1.0)
    y = np.clip(x / scale, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, float(scale)


def make_kv_fp8(w: Workload, which: str, threads: int | None = None):
    """Full [B, heads, rows, d] uint8 E4M3 codes of Q, K or V and their [B, heads] float32 scales
    (heads = H and rows = Nq for Q; the K/V head count and Nk for K and V)."""
    heads = w.H if which in ("q", "do") else w.kv_heads
    rows = w.Nq if which in ("q", "do") else w.Nk
    out = np.empty((w.B, heads, rows, w.d), dtype=np.uint8)
    scales = np.empty((w.B, heads), dtype=np.float32)
    threads = threads or min(16, len(os.sched_getaffinity(0)))

    def fill(bh):
        b, h = divmod(bh, heads)
        out[b, h], scales[b, h] = head_block_fp8(w, which, b, h)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(w.B * heads)))
    return out, scales


def head_block_f32(w: Workload, which: str, b: int, h: int) -> np.ndarray:
    """Same values as head_block, as float32 (exact for bf16 workloads)."""
    x = head_block(w, which, b, h)
    return bf16_bits_to_f32(x) if w.dtype == "bf16" else x


def make_tensor(w: Workload, which: str, threads: int | None = None) -> np.ndarray:
    """Full [B, heads, rows, d] tensor in storage form (heads = H for Q, the K/V head count for
    K and V), heads drawn in parallel."""
    rows = w.Nq if which in ("q", "do") else w.Nk
    heads = w.H if which in ("q", "do") else w.kv_heads
    out = np.empty((w.B, heads, rows, w.d), dtype=np.uint16 if w.dtype == "bf16" else np.float32)
    threads = threads or min(16, len(os.sched_getaffinity(0)))

    def fill(bh):
        b, h = divmod(bh, heads)
        out[b, h] = head_block(w, which, b, h)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(w.B * heads)))
    return out


def as_f32(w: Workload, x: np.ndarray) -> np.ndarray:
    """Storage form -> float32 values."""
    return bf16_bits_to_f32(x) if w.dtype == "bf16" else np.asarray(x, dtype=np.float32)
