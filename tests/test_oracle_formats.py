"""Pins of the oracle's format decoding and of the input generators (CPU only)."""
import numpy as np
import pytest
import torch

from oracle.formats import E4M3FN_TABLE, bf16_to_f64, e4m3fn_to_f64
from mla_paged_decode_03_amd import inputs as gen


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_bf16_decode_matches_torch_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(bf16_to_f64(bits), ref)


def test_e4m3fn_table_matches_torch_for_every_pattern():
    bits = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(e4m3fn_to_f64(bits), ref)


def test_e4m3fn_special_values():
    # OCP e4m3fn: max 448, smallest subnormal 2^-9, smallest normal 2^-6, NaN at 0x7F/0xFF, no inf
    assert E4M3FN_TABLE[0x7E] == 448.0
    assert E4M3FN_TABLE[0xFE] == -448.0
    assert E4M3FN_TABLE[0x01] == 2.0 ** -9
    assert E4M3FN_TABLE[0x08] == 2.0 ** -6
    assert E4M3FN_TABLE[0x38] == 1.0
    assert np.isnan(E4M3FN_TABLE[0x7F]) and np.isnan(E4M3FN_TABLE[0xFF])
    assert E4M3FN_TABLE[0x80] == 0.0 and np.signbit(E4M3FN_TABLE[0x80])
    assert np.all(np.isfinite(np.delete(E4M3FN_TABLE, [0x7F, 0xFF])))


def test_generator_bf16_rounding_matches_torch():
    x = gen.random_f32(7, 1, (4096,)) * np.float32(3.0)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]  # exact ties
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generator_is_deterministic_and_shaped():
    w = gen.workload("tiny")
    a = gen.generate(w)
    b = gen.generate(w)
    assert np.array_equal(a.cache, b.cache) and np.array_equal(a.q, b.q)
    assert np.array_equal(a.block_table, b.block_table)
    assert a.cache.shape == (32, 16, 576) and a.cache.dtype == np.uint16
    assert a.q.shape == (1, 16, 512) and a.q_pe.shape == (1, 16, 64)
    assert list(a.seq_lens) == [256]
    used = a.block_table[0]
    assert len(set(used.tolist())) == 16 and used.min() >= 0 and used.max() < 32


def test_generator_fp8_scale_rule():
    w = gen.workload("fp8", B=2, seed=5)
    inp = gen.generate(w, seq_lens=np.array([70, 3]))
    assert inp.cache.dtype == np.uint8
    dec = e4m3fn_to_f64(inp.cache)
    # per-tensor scale amax/448: the largest magnitude maps to 448 exactly
    assert np.nanmax(np.abs(dec)) == 448.0
    assert inp.kv_scale > 0


def test_generator_seq_len_recipes():
    import math
    lt = gen.generate(gen.workload("longtail", B=4))
    assert lt.seq_lens.min() >= 512 and lt.seq_lens.max() <= 32768
    rng = np.random.Generator(np.random.PCG64(1002))
    u = rng.uniform(math.log(512), math.log(32768), size=128)
    assert gen.draw_seq_lens(gen.workload("longtail"),
                             np.random.Generator(np.random.PCG64(1002))).tolist() == \
        np.clip(np.floor(np.exp(u)), 512, 32768).astype(int).tolist()


def test_round_to_bf16_against_torch_and_ties():
    """Nearest bfloat16, ties to even: torch's float32 -> bfloat16 conversion on random
    float32 values of many magnitudes (torch converts float64 through float32, a double
    rounding, so the comparison uses float32 inputs), and exact midpoints built by hand."""
    import torch
    from oracle.formats import round_to_bf16
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-30, 30, 200_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_to_bf16(x.astype(np.float64)), ref)
    one_ulp = 2.0 ** -7  # spacing of bfloat16 in [1, 2)
    assert round_to_bf16(np.array([1 + one_ulp / 2]))[0] == 1.0  # tie -> even (1.0)
    assert round_to_bf16(np.array([1 + 3 * one_ulp / 2]))[0] == 1 + 2 * one_ulp  # tie -> even
    assert round_to_bf16(np.array([-(1 + 3 * one_ulp / 2)]))[0] == -(1 + 2 * one_ulp)
    assert round_to_bf16(np.array([1 + one_ulp / 2 + 2.0 ** -40]))[0] == 1 + one_ulp
    assert round_to_bf16(np.array([0.0]))[0] == 0.0

