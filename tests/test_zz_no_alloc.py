"""fa_decode_noalloc (through the C ABI): the decode entry point that allocates nothing, with its
split partials in the library's fixed device scratch.

It must give what fa_decode_split_ex + fa_decode_combine give on the same inputs, bit for bit
(same kernels, same partial layout), and so match the float64 reference at the decode
tolerances.  Two calls in a row, the second with a smaller input, check that a call does not
depend on what an earlier call left in the shared scratch."""
import pytest
import torch

import exact_attention_126_amd as fa
import oracle
from synth import inputs as si
from synth.workloads import Workload
from tests.gpu_util import assert_parity, device_inputs, from_device, metrics

pytestmark = pytest.mark.gpu


def _w(name, B, H, Hkv, Nk, d, dtype, S, seed):
    return Workload(name, B=B, H=H, H_kv=Hkv, Nq=1, Nk=Nk, d=d, dtype=dtype, causal=False, seed=seed, num_splits=S,
                    k_rule=("scale_all", 2.0))


def _both(w):
    host, dev = device_inputs(w)
    print(f"  [fa_decode_noalloc] {w.name}: B={w.B} H={w.H} H_kv={w.kv_heads} Nk={w.Nk} d={w.d} {w.dtype} "
          f"splits={w.num_splits} partials {fa.fa_decode_workspace_bytes(w.B, w.H, w.d, w.num_splits)} B", flush=True)
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, 1), dtype=torch.float32, device="cuda")
    fa.fa_decode_noalloc(dev["q"], dev["k"], dev["v"], o, lse, w.num_splits, w.scale)
    torch.cuda.synchronize()
    print(f"  [fa_decode_split_ex + fa_decode_combine] {w.name}", flush=True)
    o2, l2 = fa.decode(dev["q"], dev["k"], dev["v"], w.num_splits, w.scale)
    torch.cuda.synchronize()
    return host, o, lse, o2, l2


def _check(w, host, o, lse, o2, l2):
    assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                       o2.view(torch.int16) if o2.dtype == torch.bfloat16 else o2), w.name
    assert torch.equal(lse, l2), w.name
    o_ref, l_ref = oracle.attention(si.as_f32(w, host["q"]), si.as_f32(w, host["k"]), si.as_f32(w, host["v"]),
                                    w.scale, False)
    assert_parity(w.dtype, metrics(from_device(o), from_device(lse), o_ref, l_ref), w.name)


def test_noalloc_two_calls_second_smaller():
    big = _w("noalloc_big_g4", 4, 32, 8, 8192, 128, "bf16", 64, seed=71)       # 4.3 MB of partials
    small = _w("noalloc_small_d64_f32", 1, 3, 3, 300, 64, "f32", 7, seed=72)  # 4.4 KB of partials
    first = _both(big)
    second = _both(small)
    _check(big, *first)
    _check(small, *second)


def test_noalloc_near_the_scratch_limit():
    """B8 H32 d128 with 120 splits: 16.0 MB of partials, half the scratch, then a smaller call."""
    w = _w("noalloc_s120", 8, 32, 32, 4096, 128, "bf16", 120, seed=73)
    assert fa.fa_decode_workspace_bytes(w.B, w.H, w.d, w.num_splits) <= fa.DECODE_NOALLOC_SCRATCH_BYTES
    _check(w, *_both(w))
    w2 = _w("noalloc_after_s120", 2, 2, 1, 1000, 128, "bf16", 16, seed=74)
    _check(w2, *_both(w2))


def test_noalloc_rejects_partials_beyond_the_scratch():
    w = _w("noalloc_too_big", 16, 32, 32, 512, 128, "bf16", 127, seed=75)
    assert fa.fa_decode_workspace_bytes(w.B, w.H, w.d, w.num_splits) > fa.DECODE_NOALLOC_SCRATCH_BYTES
    _, dev = device_inputs(w)
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode_noalloc(dev["q"], dev["k"], dev["v"], o, lse, w.num_splits, w.scale)
    assert e.value.status == 8
