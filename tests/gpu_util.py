"""Helpers for the GPU parity tests: device transfer of the synthetic inputs and the
tolerance checks against the float64 reference."""
from __future__ import annotations

import numpy as np
import torch

from synth import inputs as si
from synth.workloads import Workload

# Tolerances: bf16 inputs -> max-abs <= 2e-2 and relative L2 <= 5e-3 on O, max-abs <= 1e-3 on LSE;
# fp32 inputs -> relative L2 <= 1e-5 on O and max relative error <= 1e-5 on LSE.
BF16_O_MAXABS, BF16_O_RELL2, BF16_LSE_MAXABS = 2e-2, 5e-3, 1e-3
F32_O_RELL2, F32_LSE_MAXREL = 1e-5, 1e-5


def to_device(w: Workload, x: np.ndarray) -> torch.Tensor:
    if w.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def from_device(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> exact float32 numpy copy."""
    if t.dtype == torch.bfloat16:
        return si.bf16_bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.float().cpu().numpy()


def device_inputs(w: Workload):
    """(host storage arrays, device tensors) for Q, K, V."""
    host = {x: si.make_tensor(w, x) for x in "qkv"}
    return host, {x: to_device(w, host[x]) for x in "qkv"}


def metrics(o, lse, o_ref, lse_ref) -> dict:
    o, lse = np.asarray(o, np.float64), np.asarray(lse, np.float64)
    d = np.abs(o - o_ref)
    row_err = np.sqrt((d.reshape(-1, o.shape[-1]) ** 2).sum(-1))
    return {
        "o_maxabs": float(d.max()),
        "o_rel_l2": float(np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)),
        "o_worst_row_l2": float(row_err.max()),
        "lse_maxabs": float(np.abs(lse - lse_ref).max()),
        "lse_maxrel": float((np.abs(lse - lse_ref) / np.maximum(np.abs(lse_ref), 1e-30)).max()),
        "finite": bool(np.isfinite(o).all() and np.isfinite(lse).all()),
    }


def assert_parity(dtype: str, m: dict, what: str = ""):
    print(f"    parity {what}: {m}", flush=True)
    assert m["finite"], f"non-finite output {what}"
    if dtype == "bf16":
        assert m["o_maxabs"] <= BF16_O_MAXABS, (what, m)
        assert m["o_rel_l2"] <= BF16_O_RELL2, (what, m)
        assert m["lse_maxabs"] <= BF16_LSE_MAXABS, (what, m)
    else:
        assert m["o_rel_l2"] <= F32_O_RELL2, (what, m)
        assert m["lse_maxrel"] <= F32_LSE_MAXREL, (what, m)


def sample_rows(n: int, count: int, seed: int) -> np.ndarray:
    """Edge rows (first/last, around 64/128-row tile boundaries) plus random ones."""
    edges = {0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 129, 255, 256, n // 2, n - 129, n - 128, n - 65, n - 64,
             n - 2, n - 1}
    rnd = np.random.default_rng(seed).choice(n, size=min(count, n), replace=False)
    return np.array(sorted({r for r in edges if 0 <= r < n} | set(rnd.tolist())))
