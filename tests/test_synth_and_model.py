"""Input generator and work-model tests (CPU only)."""
import json
import math
import os

import numpy as np

import synth
from synth import inputs as si
import roofline as rl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_is_nearest_even():
    g = np.random.default_rng(0)
    x = (g.standard_normal(200000) * np.exp(g.uniform(-20, 20, 200000))).astype(np.float32)
    bits = si.round_to_bf16_bits(x)
    up = si.bf16_bits_to_f32(bits).astype(np.float64)
    # the neighbouring bf16 values on either side
    nb_lo = si.bf16_bits_to_f32((bits - 1).astype(np.uint16)).astype(np.float64)
    nb_hi = si.bf16_bits_to_f32((bits + 1).astype(np.uint16)).astype(np.float64)
    xd = x.astype(np.float64)
    err = np.abs(up - xd)
    assert (err <= np.abs(nb_lo - xd)).all() and (err <= np.abs(nb_hi - xd)).all()
    # explicit ties: halfway cases go to the even mantissa
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000], dtype=np.uint32).view(np.float32)
    assert list(si.round_to_bf16_bits(ties)) == [0x3F80, 0x3F82, 0xBF80, 0x4049 + 1 if (0x4049 & 1) else 0x4049]


def test_bf16_widening_exact():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = si.bf16_bits_to_f32(bits)
    finite = np.isfinite(f)
    assert np.array_equal(si.round_to_bf16_bits(f[finite]), bits[finite])


def test_inputs_deterministic_and_per_head():
    w = synth.get("batch_b4h16_n2048_d64")
    a = si.head_block(w, "q", 1, 3)
    b = si.head_block(w, "q", 1, 3)
    c = si.head_block(w, "q", 1, 4)
    assert a.dtype == np.uint16 and a.shape == (2048, 64)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert not np.array_equal(si.head_block(w, "k", 1, 3), a)


def test_make_tensor_matches_head_blocks():
    w = synth.get("tiny_f32_n128_d64")
    t = si.make_tensor(w, "v")
    assert t.dtype == np.float32 and t.shape == (1, 1, 128, 64)
    assert np.array_equal(t[0, 0], si.head_block(w, "v", 0, 0))


def test_k_rules_are_exact_powers_of_two():
    w = synth.get("prefill_b8h16_n8192_d128_causal")
    k = si.bf16_bits_to_f32(si.head_block(w, "k", 0, 0)[:64])
    base = si.bf16_bits_to_f32(si.round_to_bf16_bits(si._draw(w.seed, 1, 0, 0, w.Nk, w.d)[:64]))
    assert np.array_equal(k, base * 2)
    w = synth.get("long_b1h32_n16384_d128_causal")
    k = si.bf16_bits_to_f32(si.head_block(w, "k", 0, 5)[:130])
    base = si.bf16_bits_to_f32(si.round_to_bf16_bits(si._draw(w.seed, 1, 0, 5, w.Nk, w.d)[:130]))
    rows = np.arange(130)
    assert np.array_equal(k[rows % 64 == 0], base[rows % 64 == 0] * 8)
    assert np.array_equal(k[rows % 64 != 0], base[rows % 64 != 0])


def test_values_look_standard_normal():
    w = synth.get("batch_b4h16_n2048_d64")
    x = si.head_block_f32(w, "v", 0, 0)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def _pages():
    with open(os.path.join(GOLDEN, "page_numbers.json")) as f:
        return json.load(f)


def test_page_numbers_against_model():
    p = _pages()
    e = p["n2_at_16k"]
    assert math.isclose(rl.score_matrix_elements(e["N"]), e["elements"], rel_tol=e["rel_tol"])
    e = p["n2_at_8k"]
    assert math.isclose(rl.score_matrix_elements(e["N"]), e["mebi_elements"] * 2**20, rel_tol=e["rel_tol"])
    e = p["n2_fp16_matrix_b8_h16_n8192"]
    one_matrix = e["B"] * e["H"] * rl.score_matrix_elements(e["N"]) * e["bytes_per_elt"]
    assert math.isclose(one_matrix / 2**30, e["gib"], rel_tol=e["rel_tol"])
    e = p["standard_hbm_crossings"]
    n, d = 4096, 64
    extra = rl.standard_attention_hbm_bytes(1, 1, n, d, 1) - 4 * n * d
    assert extra == e["crossings"] * n * n
    e = p["standard_hbm_at_16k"]
    gb = rl.standard_attention_hbm_bytes(1, 1, e["N"], 128, e["bytes_per_elt"]) / 1e9
    assert math.isclose(gb, e["gb"], rel_tol=e["rel_tol"])
    e = p["causal_saving"]
    assert rl.attention_flops(1, 1, 64, 64, 8, True) == e["fraction_of_dense_flops"] * rl.attention_flops(
        1, 1, 64, 64, 8, False)


def test_headline_work_figures():
    w = synth.get(synth.PREFILL_HEADLINE)
    f = rl.attention_flops(w.B, w.H, w.Nq, w.Nk, w.d, w.causal)
    assert math.isclose(f, 2.199e12, rel_tol=1e-3)
    w = synth.get(synth.DECODE_HEADLINE)
    assert rl.decode_kv_bytes(w.B, w.H, w.Nk, w.d, 2) == 2**33
    assert math.isclose(rl.PEAK_BF16_MFMA_TFLOPS, rl.CUS * rl.CLOCK_GHZ * 4096 / 1000, rel_tol=1e-4)


def test_qblock_model_bounds():
    # causal per-Q-block model: sum over q of (q+1) blocks
    b = rl.qblock_kv_model_bytes(1, 1, 1024, 64, 2, 128, True)
    rows = sum((q + 1) * 128 for q in range(8))
    assert b == rows * 2 * 64 * 2 + 2 * 1024 * 64 * 2
    assert rl.qblock_kv_model_bytes(1, 1, 1024, 64, 2, 128, False) > b
