"""GPU parity at the largest sizes the entry points take, against the float64 oracle.

* fa_fwd_masked at its largest key count, Nk = 131072 = 2048 tiles of 64 keys (each query
  block's tile list lives in LDS, 2048 entries): a mask under which every block lists all 2048
  tiles, and one of random empty / full / partial tiles, with the exact tile lists checked.
* fa_fwd_ex, bottom-right causal: a ragged chunk of queries against a long cache of 200003 keys
  (the last key tile partial, the diagonal offset 199703).
* fa_decode_split + fa_decode_combine over 262144 cached keys in 128 splits.
* fa_bwd for the same kind of chunk against 65537 keys, with grouped heads.
* fa_fwd_masked with 2048 and 2050 query blocks: the forward ranks up to 2048 blocks by tile count
  for its schedule, and past that the blocks keep their index order.
Each case runs at a few heads, so the oracle takes seconds.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_attention_126_amd as fa
import oracle
from synth import inputs as si
from synth import masks
from synth.workloads import Workload
from tests.gpu_util import assert_parity, device_inputs, from_device, metrics
from tests.test_gpu_block_mask import _host_classification

pytestmark = pytest.mark.gpu

MAX_MASK_KEYS = 2048 * 64


def _masked_run(w, dev, allowed):
    md = torch.from_numpy(masks.pack_bits(allowed).view(np.int64)).cuda()
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_fwd_masked_workspace_bytes(w.Nq, w.Nk), dtype=torch.uint8, device="cuda")
    fa.fa_fwd_masked(dev["q"], dev["k"], dev["v"], o, lse, md, ws, w.scale)
    torch.cuda.synchronize()
    return o, lse, ws


def _check_lists(w, ws, allowed):
    n_qblk, nt = -(-w.Nq // 256), -(-w.Nk // 64)
    raw = ws.cpu().numpy()
    off_cls = (4 * n_qblk + 15) // 16 * 16
    off_lst = off_cls + (n_qblk * nt + 15) // 16 * 16
    counts = raw[:4 * n_qblk].view(np.int32)
    lists = raw[off_lst:off_lst + 2 * n_qblk * nt].view(np.uint16).reshape(n_qblk, nt)
    hc, hl = _host_classification(allowed, w.Nq, w.Nk)
    assert counts.tolist() == hc
    for qb in range(n_qblk):
        assert lists[qb, :hc[qb]].tolist() == hl[qb], qb
    return hc


@pytest.mark.parametrize("d", [64, 128])
def test_masked_max_keys_every_tile_listed(d):
    """Bottom-right window as long as the keys: every row sees all keys up to its diagonal, so
    each 256-row block lists all 2048 tiles (the last ones partial for its first rows)."""
    w = Workload(f"masked_maxkeys_window_d{d}", B=1, H=2, H_kv=1, Nq=300, Nk=MAX_MASK_KEYS, d=d, dtype="bf16",
                 causal=False, seed=201, mask_rule=("window", MAX_MASK_KEYS))
    allowed = masks.element_mask(w)
    print(f"  [fa_fwd_masked] {w.name}: Nq={w.Nq} Nk={w.Nk} visible={masks.visible_pairs(allowed)}", flush=True)
    host, dev = device_inputs(w)
    o, lse, ws = _masked_run(w, dev, allowed)
    assert _check_lists(w, ws, allowed) == [2048, 2048]
    f = {x: si.as_f32(w, host[x]) for x in "qkv"}
    o_ref, l_ref = oracle.attention(f["q"], f["k"], f["v"], w.scale, allowed=allowed)
    assert_parity("bf16", metrics(from_device(o), from_device(lse), o_ref, l_ref), w.name)


def test_masked_max_keys_random_tiles():
    w = Workload("masked_maxkeys_tiles_d128", B=1, H=2, H_kv=2, Nq=513, Nk=MAX_MASK_KEYS, d=128, dtype="bf16",
                 causal=False, seed=202, mask_rule=("tiles", 203, 64, 64, 0.3, 0.4, 0.5))
    allowed = masks.element_mask(w)
    print(f"  [fa_fwd_masked] {w.name}: Nq={w.Nq} Nk={w.Nk} visible={masks.visible_pairs(allowed)}", flush=True)
    host, dev = device_inputs(w)
    o, lse, ws = _masked_run(w, dev, allowed)
    counts = _check_lists(w, ws, allowed)
    print(f"    tiles listed per block: {counts}", flush=True)
    f = {x: si.as_f32(w, host[x]) for x in "qkv"}
    o_ref, l_ref = oracle.attention(f["q"], f["k"], f["v"], w.scale, allowed=allowed)
    og, lg = from_device(o), from_device(lse)
    empty = ~allowed.any(axis=1)
    assert np.all(og[:, :, empty] == 0.0) and np.all(np.isneginf(lg[:, :, empty]))
    vis = ~empty
    assert_parity("bf16", metrics(og[:, :, vis], lg[:, :, vis], o_ref[:, :, vis], l_ref[:, :, vis]), w.name)


def test_chunk_against_long_cache_bottom_right():
    w = Workload("chunk_nq300_nk200003_br", B=1, H=4, H_kv=1, Nq=300, Nk=200003, d=128, dtype="bf16", causal=True,
                 seed=204, causal_align="bottom_right")
    print(f"  [fa_fwd_ex] {w.name}: Nq={w.Nq} Nk={w.Nk} H={w.H} H_kv={w.kv_heads} bottom-right", flush=True)
    host, dev = device_inputs(w)
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    fa.fa_fwd_ex(dev["q"], dev["k"], dev["v"], o, lse, fa.FA_MASK_CAUSAL_BOTTOM_RIGHT, w.scale)
    torch.cuda.synchronize()
    f = {x: si.as_f32(w, host[x]) for x in "qkv"}
    o_ref, l_ref = oracle.attention(f["q"], f["k"], f["v"], w.scale, causal=True, diag=w.Nk - w.Nq)
    assert_parity("bf16", metrics(from_device(o), from_device(lse), o_ref, l_ref), w.name)


def test_decode_long_cache_many_splits():
    w = Workload("decode_b2h4_nk262144_s128", B=2, H=4, H_kv=4, Nq=1, Nk=262144, d=128, dtype="bf16",
                 causal=False, seed=205, num_splits=128)
    print(f"  [fa_decode_split + combine] {w.name}: Nk={w.Nk} splits={w.num_splits}", flush=True)
    host, dev = device_inputs(w)
    o, lse = fa.decode(dev["q"], dev["k"], dev["v"], w.num_splits, w.scale)
    torch.cuda.synchronize()
    f = {x: si.as_f32(w, host[x]) for x in "qkv"}
    o_ref, l_ref = oracle.attention(f["q"], f["k"], f["v"], w.scale)
    assert_parity("bf16", metrics(from_device(o), from_device(lse).reshape(l_ref.shape), o_ref, l_ref), w.name)


def test_bwd_chunk_against_long_cache():
    """fa_bwd for a bottom-right chunk of 300 queries against 65537 keys (the last key tile
    partial), grouped heads, against the reference and the per-element bounds."""
    from tests import bwd_bounds
    from tests.test_gpu_bwd import _inputs as bwd_inputs, _run as bwd_run, _w as bwd_w
    w = bwd_w("bwd_nq300_nk65537_br_g2", 1, 4, 2, 300, 65537, 128, "bottom_right", seed=206)
    host, dev = bwd_inputs(w)
    (dq, dk, dv), (o, lse) = bwd_run(w, dev, with_forward=True)
    f = {x: si.as_f32(w, host[x]) for x in host}
    res = bwd_bounds.reference_and_bounds(f["q"], f["k"], f["v"], f["do"], from_device(o), from_device(lse), w.scale,
                                          w.causal, w.diag)
    bwd_bounds.check({"dq": from_device(dq), "dk": from_device(dk), "dv": from_device(dv)}, res, w.name)


def _block_tile_mask(nq, nk, seed, p_empty=0.3, p_full=0.3):
    """Each (256-row block, 64-key tile) empty, full, or bit by bit at random (seeded); built with
    broadcasting so that half a million rows take seconds."""
    g = np.random.default_rng(seed)
    nqb, nt = -(-nq // 256), -(-nk // 64)
    cls = g.choice(3, size=(nqb, nt), p=[p_empty, p_full, 1.0 - p_empty - p_full]).astype(np.int8)
    big = cls[np.arange(nq) // 256][:, np.arange(nk) // 64]
    bits = g.integers(0, 2, size=(nq, nk), dtype=np.uint8).astype(bool)
    return (big == 1) | ((big == 2) & bits)


@pytest.mark.parametrize("n_blocks", [2048, 2050])
def test_masked_block_count_at_and_past_the_ranked_limit(n_blocks):
    """Random empty / full / partial (256-row block, 64-key tile) classes, so the blocks' tile counts
    differ; 2048 blocks are all ranked for the heaviest-first schedule, 2050 keep index order (the
    last block ragged).  Every row against the reference."""
    nq = (n_blocks - 1) * 256 + 77
    w = Workload(f"masked_{n_blocks}_blocks_nk100_d64", B=1, H=1, H_kv=1, Nq=nq, Nk=100, d=64, dtype="bf16",
                 causal=False, seed=207)
    allowed = _block_tile_mask(w.Nq, w.Nk, 208)
    print(f"  [fa_fwd_masked] {w.name}: Nq={w.Nq} Nk={w.Nk} blocks={n_blocks} visible={masks.visible_pairs(allowed)}",
          flush=True)
    host, dev = device_inputs(w)
    o, lse, _ = _masked_run(w, dev, allowed)
    f = {x: si.as_f32(w, host[x]) for x in "qkv"}
    o_ref, l_ref = oracle.attention(f["q"], f["k"], f["v"], w.scale, allowed=allowed)
    og, lg = from_device(o), from_device(lse)
    empty = ~allowed.any(axis=1)
    assert np.all(og[:, :, empty] == 0.0) and np.all(np.isneginf(lg[:, :, empty]))
    vis = ~empty
    assert_parity("bf16", metrics(og[:, :, vis], lg[:, :, vis], o_ref[:, :, vis], l_ref[:, :, vis]), w.name)
