"""Parity of split-KV decode (fa_decode_split + fa_decode_combine through the C ABI) with the
float64 reference: the per-split partials, the combine alone on reference partials, and the
final output, at small shapes (ragged and empty splits).  The full decode workload is compared
on every head in tests/test_gpu_workloads_all_heads.py."""
import numpy as np
import pytest
import torch

import exact_attention_126_amd as fa
import oracle
from synth import inputs as si
from synth.workloads import Workload
from tests.gpu_util import assert_parity, device_inputs, from_device, metrics

pytestmark = pytest.mark.gpu


def _w(name, B, H, Nk, d, dtype, S, k_rule=("none",), seed=11):
    return Workload(name, B=B, H=H, Nq=1, Nk=Nk, d=d, dtype=dtype, causal=False, seed=seed, k_rule=k_rule,
                    num_splits=S)


SMALL = [
    _w("nk1_s1", 1, 1, 1, 128, "bf16", 1),
    _w("nk100_s64_empty_tail", 2, 3, 100, 128, "bf16", 64),
    _w("nk1000_s3_uneven", 1, 2, 1000, 64, "bf16", 3),
    _w("nk37_s37", 1, 1, 37, 128, "bf16", 37),
    _w("nk4096_s16_k2", 2, 2, 4096, 128, "bf16", 16, ("scale_all", 2.0)),
    _w("nk777_s5_rows8", 1, 3, 777, 64, "bf16", 5, ("scale_rows_every", 64, 8.0)),
    _w("f32_nk300_s7", 2, 2, 300, 128, "f32", 7),
    _w("f32_nk65_s64", 1, 1, 65, 64, "f32", 64),
]


def _split_and_combine(w, dev):
    print(f"  [fa_decode] {w.name}: B={w.B} H={w.H} Nk={w.Nk} d={w.d} {w.dtype} splits={w.num_splits}", flush=True)
    ws = fa.decode_workspace(dev["q"], w.num_splits)
    fa.fa_decode_split(dev["q"], dev["k"], dev["v"], ws, w.num_splits, w.scale)
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, 1), dtype=torch.float32, device="cuda")
    fa.fa_decode_combine(ws, o, lse, w.num_splits)
    torch.cuda.synchronize()
    return ws, o, lse


def _unpack_ws(w, ws):
    n = w.B * w.H * w.num_splits
    flat = ws.cpu().numpy()
    return flat[: n * w.d].reshape(w.B, w.H, w.num_splits, w.d), flat[n * w.d: n * (w.d + 2)].reshape(
        w.B, w.H, w.num_splits, 2)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_decode_small(w):
    host, dev = device_inputs(w)
    ws, o, lse = _split_and_combine(w, dev)
    q, k, v = (si.as_f32(w, host[x]) for x in "qkv")
    o_ref, l_ref = oracle.attention(q, k, v, w.scale, False)
    assert_parity(w.dtype, metrics(from_device(o), from_device(lse), o_ref, l_ref), w.name)
    # the partials themselves (float32 state of each split)
    o_part, ml = _unpack_ws(w, ws)
    for b in range(w.B):
        for h in range(w.H):
            po, pm, pl = oracle.split_partials(q[b, h, 0], k[b, h], v[b, h], w.scale, w.num_splits)
            empty = np.isneginf(pm)
            assert np.array_equal(np.isneginf(ml[b, h, :, 0]), empty)
            assert np.all(ml[b, h, empty, 1] == 0) and np.all(o_part[b, h, empty] == 0)
            ne = ~empty
            assert np.abs(ml[b, h, ne, 0] - pm[ne]).max() < 1e-5 * max(1.0, np.abs(pm[ne]).max())
            # l and O_part are relative to each split's max: compare relative to the reference
            assert np.abs(ml[b, h, ne, 1] / pl[ne] - 1).max() < 1e-4
            scale_o = np.abs(po[ne]).max() + 1e-30
            assert np.abs(o_part[b, h, ne] - po[ne]).max() / scale_o < 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_combine_on_reference_partials(dtype):
    """fa_decode_combine alone: float32 partials computed by the reference, merged on the GPU."""
    w = _w("combine_only", 2, 3, 500, 128, dtype, 9, ("scale_all", 2.0))
    host, _ = device_inputs(w)
    q, k, v = (si.as_f32(w, host[x]) for x in "qkv")
    n = w.B * w.H * w.num_splits
    o_part = np.zeros((w.B, w.H, w.num_splits, w.d), np.float32)
    ml = np.zeros((w.B, w.H, w.num_splits, 2), np.float32)
    o_ref = np.zeros((w.B, w.H, 1, w.d))
    l_ref = np.zeros((w.B, w.H, 1))
    for b in range(w.B):
        for h in range(w.H):
            po, pm, pl = oracle.split_partials(q[b, h, 0], k[b, h], v[b, h], w.scale, w.num_splits)
            o_part[b, h], ml[b, h, :, 0], ml[b, h, :, 1] = po, pm, pl
            o_ref[b, h, 0], l_ref[b, h, 0] = oracle.combine_partials(po.astype(np.float32), pm.astype(np.float32),
                                                                     pl.astype(np.float32))
    ws = torch.from_numpy(np.concatenate([o_part.reshape(-1), ml.reshape(-1)])).cuda()
    assert ws.numel() == n * (w.d + 2)
    o = torch.empty((w.B, w.H, 1, w.d), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H, 1), dtype=torch.float32, device="cuda")
    print(f"  [fa_decode_combine] reference partials {dtype}", flush=True)
    fa.fa_decode_combine(ws, o, lse, w.num_splits)
    torch.cuda.synchronize()
    assert_parity(dtype, metrics(from_device(o), from_device(lse), o_ref, l_ref), "combine only")
