"""Pins of the oracle's static fp8 query quantisation (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quant as Q


def _finite_codes():
    return np.array([c for c in range(256) if not np.isnan(F.E4M3FN_TABLE[c])], dtype=np.uint8)


def test_every_finite_code_round_trips():
    codes = _finite_codes()
    vals = F.E4M3FN_TABLE[codes].astype(np.float32)
    enc = Q.encode_e4m3fn(vals)
    for c, e, v in zip(codes, enc, vals):
        assert e == c or (v == 0 and F.E4M3FN_TABLE[e] == 0 and np.signbit(F.E4M3FN_TABLE[e]) == np.signbit(v))


def test_midpoints_round_to_the_even_code():
    pos = sorted(set(F.E4M3FN_TABLE[c] for c in range(0, 0x7F)))  # 0 .. 448
    lo, hi = np.array(pos[:-1]), np.array(pos[1:])
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (lo + hi) / 2)  # midpoints are exact in float32
    got = F.E4M3FN_TABLE[Q.encode_e4m3fn(mid)]
    lo_code = Q.encode_e4m3fn(lo.astype(np.float32))
    hi_code = Q.encode_e4m3fn(hi.astype(np.float32))
    want = np.where(lo_code % 2 == 0, lo, hi)
    assert np.all(got == want)
    assert np.all(np.where(lo_code % 2 == 0, lo_code, hi_code) % 2 == 0)
    # just below / above a midpoint go to the nearer neighbour
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    assert np.all(F.E4M3FN_TABLE[Q.encode_e4m3fn(below)] == lo)
    assert np.all(F.E4M3FN_TABLE[Q.encode_e4m3fn(above[:-1])] == hi[:-1])


def test_negative_values_mirror_positive_ones():
    x = np.random.default_rng(3).uniform(0, 448, 5000).astype(np.float32)
    assert np.all(Q.encode_e4m3fn(-x) == (Q.encode_e4m3fn(x) | 0x80))


def test_agrees_with_torch_float8_conversion():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-14, 6, 100000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(Q.encode_e4m3fn(x), ref)


def test_quantize_is_within_half_a_grid_step_and_saturates():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000).astype(np.float32) * 3
    for q_scale in (1.0, 0.0123, 5.0 / 448):
        y = (x.astype(np.float64) / q_scale)
        codes = Q.quantize(x, q_scale)
        v = F.E4M3FN_TABLE[codes]
        inside = np.abs(y) < 440
        # grid step at |v|: 2^(e-3) for normals, 2^-9 for subnormals
        e = np.floor(np.log2(np.maximum(np.abs(v[inside]), 2.0 ** -6)))
        step = 2.0 ** (e - 3)
        assert np.all(np.abs(v[inside] - y[inside]) <= step / 2 * (1 + 1e-6) + 1e-7 * np.abs(y[inside]))
        big = np.abs(y) > 460
        assert np.all(np.abs(v[big]) == 448.0)


def test_concat_layout():
    rng = np.random.default_rng(2)
    ql = rng.integers(0, 1 << 16, size=(2, 3, 512), dtype=np.uint16) & 0x3FFF  # finite, moderate
    qp = rng.integers(0, 1 << 16, size=(2, 3, 64), dtype=np.uint16) & 0x3FFF
    q8 = Q.concat_quant_q(ql, qp, 0.5)
    assert q8.shape == (2, 3, 576) and q8.dtype == np.uint8
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(q8[..., :512], Q.quantize(f(ql), 0.5))
    assert np.array_equal(q8[..., 512:], Q.quantize(f(qp), 0.5))


def test_rejects_values_outside_the_range():
    with pytest.raises(ValueError):
        Q.encode_e4m3fn(np.array([449.0], np.float32))
