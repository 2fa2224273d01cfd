"""Pins of oracle/bmm8.py (fp8 W_UK / W_UV BMMs): the weight quantisation's steps against
torch's own bf16 arithmetic and float8 conversion, the quantisation invariants (the
largest element lands on 448, reconstruction within half an e4m3 step), the product
against brute-force loops, exactness when every value is representable, and the
absorption / up-projection against the bf16 definitions within fp8 precision."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import bmm8 as Q8
from oracle.formats import E4M3FN_TABLE, bf16_to_f64


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("kind", ["uk", "uv"])
def test_weight_quant_steps_against_torch(kind):
    """Each step of the per-tensor weight quantisation against torch's primitives: bf16
    tensor arithmetic (float32 compute, bf16 rounding) and the float8_e4m3fn cast."""
    rng = np.random.default_rng(1)
    Wb = _bf16_bits(rng.standard_normal((64, 3, 16)) * 0.02)
    codes, w_scale = Q8.quant_weight(Wb, kind)
    Wt = torch.from_numpy(Wb.view(np.int16)).view(torch.bfloat16)
    amax = Wt.abs().max()
    s = torch.tensor(448.0, dtype=torch.bfloat16) / amax  # bf16 op: float32 compute, bf16 result
    y = (Wt * s).clamp(-448, 448)
    ref = y.float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref = ref.transpose(1, 0, 2) if kind == "uk" else ref.transpose(1, 2, 0)
    assert np.array_equal(codes, ref)
    assert w_scale == (1.0 / s.float()).item()  # torch's float32 reciprocal of the bf16 scale


def test_weight_quant_invariants_and_layout():
    rng = np.random.default_rng(2)
    Wb = _bf16_bits(rng.standard_normal((32, 4, 8)) * 0.02)
    W = bf16_to_f64(Wb)
    ck, sk = Q8.quant_weight(Wb, "uk")
    cv, sv = Q8.quant_weight(Wb, "uv")
    assert ck.shape == (4, 32, 8) and cv.shape == (4, 8, 32) and sk == sv
    l, h, p = np.unravel_index(np.argmax(np.abs(W)), W.shape)
    assert abs(E4M3FN_TABLE[ck[h, l, p]]) == 448.0
    for (l, h, p) in [(0, 0, 0), (31, 3, 7), (5, 2, 1)]:
        assert ck[h, l, p] == cv[h, p, l]
    rec = E4M3FN_TABLE[ck].transpose(1, 0, 2) * np.float64(sk)
    big = np.abs(W) >= 2.0 ** -6 / 448 * np.abs(W).max() * 8  # away from the subnormal range
    # half an e4m3 step (2^-4 relative), plus the bf16 rounding of W * s before it
    assert np.all(np.abs(rec - W)[big] <= (2.0 ** -4 + 2.0 ** -8) * np.abs(W)[big])


def test_act_quant_invariants():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((5, 384)).astype(np.float32) * np.float32(3.0)
    a[2, 128:256] = 0.0
    codes, d = Q8.quant_act(a)
    assert codes.shape == a.shape and d.shape == (5, 3)
    val = E4M3FN_TABLE[codes].reshape(5, 3, 128)
    g = a.reshape(5, 3, 128)
    for m in range(5):
        for j in range(3):
            if not np.any(g[m, j]):
                assert not np.any(codes.reshape(5, 3, 128)[m, j])
                continue
            i = np.argmax(np.abs(g[m, j]))
            assert abs(val[m, j, i]) == 448.0
            rec = val[m, j] * np.float64(d[m, j])
            big = np.abs(g[m, j]) >= np.abs(g[m, j]).max() * 2.0 ** -6
            assert np.all(np.abs(rec - g[m, j])[big] <= 2.0 ** -4 * np.abs(g[m, j])[big] * (1 + 1e-6))


def test_bmm_brute_force():
    rng = np.random.default_rng(4)
    H, M, Nn, K = 2, 3, 4, 256
    Ac = rng.integers(0, 256, (H, M, K), dtype=np.uint8)
    Wc = rng.integers(0, 256, (H, Nn, K), dtype=np.uint8)
    for c in (Ac, Wc):
        c[(c & 0x7F) == 0x7F] = 0  # no NaN codes
    d = rng.random((H, M, K // 128)).astype(np.float32)
    ws = np.float32(0.37)
    C = Q8.bmm(Ac, d, Wc, ws)
    for h in range(H):
        for m in range(M):
            for n in range(Nn):
                ref = 0.0
                for g in range(K // 128):
                    part = sum(E4M3FN_TABLE[Ac[h, m, k]] * E4M3FN_TABLE[Wc[h, n, k]] for k in range(128 * g, 128 * g + 128))
                    ref += float(d[h, m, g]) * part
                assert abs(C[h, m, n] - ref * float(ws)) <= 1e-9 * max(1.0, abs(ref))


def test_exact_when_every_value_is_representable():
    """Weights and activations built from e4m3 values whose groups peak at 448 / 2^j: the
    scales are powers of two and nothing rounds, so the fp8 absorption equals the plain
    product of the inputs."""
    rng = np.random.default_rng(5)
    grid = E4M3FN_TABLE[np.arange(256)]
    grid = grid[np.isfinite(grid)]
    T, N, P, Lkv = 3, 2, 128, 64
    q = rng.choice(grid, (T, N, P)) / 2.0 ** 3
    q[:, :, 7] = 448.0 / 2.0 ** 3  # each (token, head) group peaks at 448 / 8
    W = rng.choice(grid[np.abs(grid) >= 2.0 ** -3], (Lkv, N, P)) / 2.0 ** 10
    W[0, 0, 0] = 448.0 / 2.0 ** 10
    qb, Wb = _bf16_bits(q), _bf16_bits(W)
    assert np.array_equal(bf16_to_f64(qb), q) and np.array_equal(bf16_to_f64(Wb), W)
    codes, ws = Q8.quant_weight(Wb, "uk")
    assert ws == np.float32(2.0 ** -10)
    got = Q8.absorb_fp8(qb, codes, ws)
    assert np.array_equal(got, A.absorb(q, W))


def test_absorb_and_up_within_fp8_precision():
    rng = np.random.default_rng(6)
    T, N, P, Lkv, V = 4, 3, 128, 256, 128
    qb = _bf16_bits(rng.standard_normal((T, N, P)))
    ob = _bf16_bits(rng.standard_normal((T, N, Lkv)) * 0.1)
    Wk = _bf16_bits(rng.standard_normal((Lkv, N, P)) * 0.02)
    Wv = _bf16_bits(rng.standard_normal((Lkv, N, V)) * 0.02)
    ck, sk = Q8.quant_weight(Wk, "uk")
    cv, sv = Q8.quant_weight(Wv, "uv")
    for got, ref in ((Q8.absorb_fp8(qb, ck, sk), A.absorb(bf16_to_f64(qb), bf16_to_f64(Wk))),
                     (Q8.up_fp8(ob, cv, sv), A.up_proj(bf16_to_f64(ob), bf16_to_f64(Wv)))):
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert 1e-3 < rel < 0.05  # fp8 operands: a few per cent, and not exact
