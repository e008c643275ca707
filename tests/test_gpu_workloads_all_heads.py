"""Parity of every head of the full-size workloads with the float64 reference, element by element.

Each workload is launched once, through the C ABI, with the entry point and launch
configuration the benchmark times.  The reference runs on every (batch, head) in the forked
worker pool (tests/oracle_pool.py), and the whole output tensor is held to the tolerances:
  bf16: max-abs <= 2e-2 and relative L2 <= 5e-3 on O, max-abs <= 1e-3 on LSE;
  fp32: relative L2 <= 1e-5 on O, max relative error <= 1e-5 on LSE.
The same bars are checked again on the edge rows of every head (first and last rows, rows
around the 32-, 64-, 128- and 256-row boundaries), so that an error confined to a block
boundary is not averaged away in the whole-tensor norm.

Every work item of the persistent forward grid is covered, including the XCD item ranges, the
paired second block of a causal item and the cross-block prefetch, since every query row of
every head is compared.

The reference takes about a second per 8192 x 8192 head on one host core, so the two largest
workloads carry a longer time limit; the comparison prints its progress while it runs."""
import pytest
import torch

import exact_attention_126_amd as fa
import synth
from synth.workloads import Workload
from tests.gpu_util import assert_parity, device_inputs, from_device
from tests.oracle_pool import compare_every_head

pytestmark = pytest.mark.gpu


def _check(w, o, lse):
    whole, edges, worst = compare_every_head(w, from_device(o), from_device(lse))
    print(f"    {w.name}: every head {whole}; worst head b={worst[0]} h={worst[1]} max-abs {worst[2]:.3e}", flush=True)
    assert whole["heads"] == w.B * w.H
    assert_parity(w.dtype, whole, f"{w.name} every head")
    assert_parity(w.dtype, edges, f"{w.name} edge rows of every head")


def _forward(w):
    _, dev = device_inputs(w)
    mask = fa.FA_MASK_NONE
    if w.causal:
        mask = fa.FA_MASK_CAUSAL_BOTTOM_RIGHT if w.causal_align == "bottom_right" else fa.FA_MASK_CAUSAL
    entry = "fa_fwd" if (w.kv_heads == w.H and w.causal_align == "top_left") else "fa_fwd_ex"
    print(f"  [{entry}] {w.name}: B={w.B} H={w.H} H_kv={w.kv_heads} Nq={w.Nq} Nk={w.Nk} d={w.d} {w.dtype} "
          f"mask={mask} seed={w.seed}", flush=True)
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    if entry == "fa_fwd":
        fa.fa_fwd(dev["q"], dev["k"], dev["v"], o, lse, w.causal, w.scale)
    else:
        fa.fa_fwd_ex(dev["q"], dev["k"], dev["v"], o, lse, mask, w.scale)
    torch.cuda.synchronize()
    return o, lse


def _decode(w):
    _, dev = device_inputs(w)
    print(f"  [fa_decode_split{'_ex' if w.kv_heads != w.H else ''} + fa_decode_combine] {w.name}: B={w.B} H={w.H} "
          f"H_kv={w.kv_heads} Nk={w.Nk} d={w.d} splits={w.num_splits} seed={w.seed}", flush=True)
    o, lse = fa.decode(dev["q"], dev["k"], dev["v"], w.num_splits, w.scale)
    torch.cuda.synchronize()
    return o, lse


def test_tiny_f32_every_row(oracle_pool):
    """B1 H1 N128 d64 fp32."""
    w = synth.get("tiny_f32_n128_d64")
    _check(w, *_forward(w))


def test_short_batch_every_head(oracle_pool):
    """B4 H16 N2048 d64, non-causal: all 64 heads."""
    w = synth.get("batch_b4h16_n2048_d64")
    _check(w, *_forward(w))


@pytest.mark.timeout(900)
def test_headline_prefill_every_head(oracle_pool):
    """B8 H16 N8192 d128 causal, K x2: all 128 heads."""
    w = synth.get("prefill_b8h16_n8192_d128_causal")
    _check(w, *_forward(w))


@pytest.mark.timeout(900)
def test_long_context_every_head(oracle_pool):
    """B1 H32 N16384 d128 causal, every 64th key row x8: all 32 heads."""
    w = synth.get("long_b1h32_n16384_d128_causal")
    _check(w, *_forward(w))


def test_decode_every_head(oracle_pool):
    """B16 H32 Nk32768 d128, 64-way split + combine: all 512 heads."""
    w = synth.get("decode_b16h32_nk32768_d128")
    _check(w, *_decode(w))


def test_chunked_prefill_every_head(oracle_pool):
    """B1 H32 H_kv8 Nq2048 Nk16384 d128, bottom-right causal (fa_fwd_ex): all 32 query heads."""
    w = synth.get("chunk_prefill_b1h32kv8_nq2048_nk16384_d128")
    _check(w, *_forward(w))


def test_grouped_decode_every_head(oracle_pool):
    """B16 H32 H_kv8 Nk32768 d128, 64-way split (fa_decode_split_ex) + combine: all 512 query heads."""
    w = synth.get("decode_gqa_b16h32kv8_nk32768_d128")
    _check(w, *_decode(w))


def _fw(name, B, H, Hkv, Nq, Nk, d, align, seed):
    return Workload(name, B=B, H=H, H_kv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype="bf16", causal=align is not None, seed=seed,
                    causal_align=align or "top_left")


# Shapes where each workgroup of the persistent forward walks several query blocks in sequence, with
# odd and even tile counts (a block with an even count loads the next block's first K tile; an odd
# count leaves the next block to load its own), with and without the rotated non-causal tile order.
SEQUENCES = [
    _fw("seq_none_nk900_odd", 2, 40, 40, 2048, 900, 128, None, seed=51),
    _fw("seq_none_nk1024_even", 2, 40, 20, 2048, 1024, 128, None, seed=52),
    _fw("seq_tl_nq2048_nk900_mixed", 4, 32, 8, 2048, 900, 128, "top_left", seed=53),
    _fw("seq_br_nq2048_nk2080_odd", 4, 32, 8, 2048, 2080, 128, "bottom_right", seed=54),
    _fw("seq_br_nq2048_nk2144_even_d64", 4, 32, 8, 2048, 2144, 64, "bottom_right", seed=55),
]


@pytest.mark.parametrize("w", SEQUENCES, ids=lambda w: w.name)
def test_block_sequences_every_head(w, oracle_pool):
    """More query blocks than compute units (fa_fwd_ex): every head."""
    o, lse = _forward(w)
    _check(w, o, lse)
