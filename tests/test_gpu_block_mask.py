"""Parity of the forward with an arbitrary element mask (fa_fwd_masked through the C ABI) with the
float64 reference on the same boolean mask (oracle.attention_head's `allowed`).

The mask rule is the Day-21 page's §6 table, last row: tiles the mask leaves empty for a whole
query block are skipped, partly visible tiles are masked element by element.  Cases:
  * random empty / full / bit-by-bit tiles at granularities that do not line up with the
    kernel's 256-query blocks and 64-key tiles, ragged Nq and Nk, grouped heads, d = 64 and 128;
  * rows with no visible key (O = 0 and LSE = -inf exactly), whole 256-row blocks without any
    visible key, and a mask that hides everything;
  * a causal sliding window and packed documents;
  * the lower-triangle mask, which must give bit for bit what fa_fwd gives with causal = 1 at
    d = 128 (the same 64-key tiles in the same order, the diagonal tiles masked element by element
    either way); at d = 64 fa_fwd runs 128-key tiles, which group the online softmax differently,
    so there both are held to the reference instead;
  * the classification pass itself: the per-block tile lists it leaves in the workspace equal a
    classification computed on the host from the boolean mask (integer work: exact);
  * the full-size packed-document workload, every head, as the benchmark times it;
  * bitwise determinism under the dynamic (block, head) schedule.
Tolerances are the bf16 bars of the forward tests."""
import numpy as np
import pytest
import torch

import exact_attention_126_amd as fa
import oracle
import synth
from synth import inputs as si
from synth import masks
from synth.workloads import Workload
from tests.gpu_util import assert_parity, device_inputs, from_device, metrics
from tests.oracle_pool import compare_every_head

pytestmark = pytest.mark.gpu


def _w(name, B, H, Hkv, Nq, Nk, d, rule, seed=61):
    return Workload(name, B=B, H=H, H_kv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype="bf16", causal=False, seed=seed,
                    mask_rule=rule)


SMALL = [
    _w("tiles32_n300_d128", 1, 2, 2, 300, 300, 128, ("tiles", 1, 32, 32)),
    _w("tiles16x48_nq513_nk1000_d64_g2", 1, 4, 2, 513, 1000, 64, ("tiles", 2, 16, 48)),
    _w("tiles64_nq700_nk2000_d128", 2, 2, 1, 700, 2000, 128, ("tiles", 3, 64, 64, 0.5, 0.2, 0.3)),
    _w("bits_nq257_nk333_d128", 1, 2, 2, 257, 333, 128, ("tiles", 4, 1, 1000, 0.0, 0.0, 0.5)),
    _w("window300_nq700_nk1500_d128", 1, 2, 2, 700, 1500, 128, ("window", 300)),
    _w("window1_n200_d64", 1, 2, 2, 200, 200, 64, ("window", 1)),
    _w("docs_n1000_d64", 1, 3, 3, 1000, 1000, 64, ("documents", 5, 40, 400)),
    _w("tiles_nq1_nk500", 1, 2, 2, 1, 500, 128, ("tiles", 6, 1, 64)),
    # more (block, head) items than compute units, a multiple of 8: every workgroup walks several
    # blocks of different tile counts in sequence
    _w("docs_b2h64_n2048_seq", 2, 64, 16, 2048, 2048, 64, ("documents", 8, 100, 900)),
    _w("tiles_b4h40_n1300_seq", 4, 40, 40, 1300, 1300, 128, ("tiles", 9, 96, 80)),
]


def _mask_dev(allowed):
    return torch.from_numpy(masks.pack_bits(allowed).view(np.int64)).cuda()


def _run(w, dev, allowed):
    print(f"  [fa_fwd_masked] {w.name}: B={w.B} H={w.H} H_kv={w.kv_heads} Nq={w.Nq} Nk={w.Nk} d={w.d} "
          f"rule={w.mask_rule} visible={masks.visible_pairs(allowed)} seed={w.seed}", flush=True)
    md = _mask_dev(allowed)
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_fwd_masked_workspace_bytes(w.Nq, w.Nk), dtype=torch.uint8, device="cuda")
    fa.fa_fwd_masked(dev["q"], dev["k"], dev["v"], o, lse, md, ws, w.scale)
    torch.cuda.synchronize()
    return o, lse, ws


def _compare(w, host, o, lse, allowed, what):
    f = {x: si.as_f32(w, host[x]) for x in "qkv"}
    o_ref, l_ref = oracle.attention(f["q"], f["k"], f["v"], w.scale, allowed=allowed)
    og, lg = from_device(o), from_device(lse)
    empty = ~allowed.any(axis=1)
    assert np.all(og[:, :, empty] == 0.0), "rows without a visible key: O = 0"
    assert np.all(np.isneginf(lg[:, :, empty])), "rows without a visible key: LSE = -inf"
    vis = ~empty
    if vis.any():
        assert_parity("bf16", metrics(og[:, :, vis], lg[:, :, vis], o_ref[:, :, vis], l_ref[:, :, vis]), what)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_masked_small(w):
    allowed = masks.element_mask(w)
    host, dev = device_inputs(w)
    o, lse, _ = _run(w, dev, allowed)
    _compare(w, host, o, lse, allowed, w.name)


def test_masked_empty_rows_and_blocks():
    """Rows 5, 77 and the whole second 256-row block see no key; so does every row of the last
    (ragged) block but one."""
    w = _w("empty_rows_blocks", 1, 2, 1, 800, 900, 128, ("tiles", 7, 8, 8))
    allowed = masks.element_mask(w)
    allowed[[5, 77]] = False
    allowed[256:512] = False
    allowed[768:] = False
    allowed[790, 899] = True
    host, dev = device_inputs(w)
    o, lse, _ = _run(w, dev, allowed)
    _compare(w, host, o, lse, allowed, w.name)


def test_masked_nothing_visible():
    w = _w("nothing_visible", 2, 2, 2, 300, 200, 64, ("window", 1))
    allowed = np.zeros((300, 200), bool)
    _, dev = device_inputs(w)
    o, lse, _ = _run(w, dev, allowed)
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("d", [64, 128])
def test_triangle_mask_equals_causal(d):
    w = _w(f"tril_n1000_d{d}", 1, 3, 3, 1000, 1000, d, ("window", 1000))
    allowed = np.tril(np.ones((1000, 1000), bool))
    host, dev = device_inputs(w)
    o, lse, _ = _run(w, dev, allowed)
    o2 = torch.empty_like(o)
    l2 = torch.empty_like(lse)
    print("  [fa_fwd] causal, same inputs", flush=True)
    fa.fa_fwd(dev["q"], dev["k"], dev["v"], o2, l2, True, w.scale)
    torch.cuda.synchronize()
    if d == 128:
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)
    else:
        _compare(w, host, o, lse, allowed, w.name + " masked")
        _compare(w, host, o2, l2, allowed, w.name + " causal")


def _host_classification(allowed, nq, nk, br=256):
    nt = -(-nk // 64)
    counts, lists = [], []
    for qb in range(-(-nq // br)):
        rows = allowed[qb * br:min(nq, qb * br + br)]
        lst = []
        for t in range(nt):
            blk = rows[:, 64 * t:min(nk, 64 * t + 64)]
            if blk.any():
                lst.append(t | (0 if blk.all() else 0x8000))
        counts.append(len(lst))
        lists.append(lst)
    return counts, lists


@pytest.mark.parametrize("w", [SMALL[0], SMALL[2], SMALL[4], SMALL[6]], ids=lambda w: w.name)
def test_tile_classification_exact(w):
    allowed = masks.element_mask(w)
    _, dev = device_inputs(w)
    _, _, ws = _run(w, dev, allowed)
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


def test_documents_workload_every_head(oracle_pool):
    """B4 H16 N8192 d128, packed documents of 256-3072 tokens, causal inside each: all 64 heads."""
    w = synth.get("masked_docs_b4h16_n8192_d128")
    allowed = masks.element_mask(w)
    _, dev = device_inputs(w)
    o, lse, _ = _run(w, dev, allowed)
    whole, edges, worst = compare_every_head(w, from_device(o), from_device(lse))
    print(f"    {w.name}: every head {whole}; worst head b={worst[0]} h={worst[1]} max-abs {worst[2]:.3e}", flush=True)
    assert whole["heads"] == w.B * w.H
    assert_parity("bf16", whole, f"{w.name} every head")
    assert_parity("bf16", edges, f"{w.name} edge rows of every head")


def test_masked_dynamic_schedule_is_deterministic():
    """The (block, head) items are claimed dynamically, so which workgroup runs a block changes from
    run to run; a block's result must not: four runs with four times more items than workgroups
    give the same bits."""
    w = _w("docs_b2h64_n2048_det", 2, 64, 16, 2048, 2048, 64, ("documents", 8, 100, 900))
    allowed = masks.element_mask(w)
    _, dev = device_inputs(w)
    runs = []
    for _ in range(4):
        o, lse, _ = _run(w, dev, allowed)
        runs.append((o, lse))
    for o, lse in runs[1:]:
        assert torch.equal(o.view(torch.int16), runs[0][0].view(torch.int16))
        assert torch.equal(lse, runs[0][1])
