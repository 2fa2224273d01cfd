"""GPU parity of the fp8 W_UK / W_UV BMMs against oracle/bmm8.py.

The weight quantisation is compared bit for bit (codes in the per-head layouts and the
dequantisation scale); the absorption and the up-projection against the oracle's fp8
product (the same quantisation decisions, taken in float32 on both sides), at ragged
token counts and at the verify workload's size (T = 128, N = 128, P = V = 128).
Tolerance: the bf16 output bounds (max-abs 1e-2, rel-L2 5e-3) and, since only the
accumulation order and the final rounding differ, 2^-7 relative per element.
"""
import numpy as np
import pytest

from tests._lib import O_MAX_ABS, O_REL_L2, bf16_dev, bf16_host, ensure_built, metrics

pytestmark = pytest.mark.gpu
ensure_built()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    return torch


def _bits(rng, shape, s=1.0):
    from mla_paged_decode_03_amd.inputs import f32_to_bf16_bits
    return f32_to_bf16_bits((rng.standard_normal(shape) * s).astype(np.float32))


def _quant(torch, Wb, which):
    from mla_paged_decode_03_amd import api
    Lkv, N, X = Wb.shape
    W8 = torch.empty((N, Lkv, X) if which == "uk" else (N, X, Lkv), dtype=torch.uint8, device="cuda")
    ws = torch.empty(1, dtype=torch.float32, device="cuda")
    api.mla_quant_weight_fp8(bf16_dev(Wb), which, W8, ws)
    torch.cuda.synchronize()
    return W8, ws


@pytest.mark.parametrize("which", ["uk", "uv"])
@pytest.mark.parametrize("N", [3, 128])
def test_quant_weight_bit_exact(torch_cuda, which, N):
    from oracle import bmm8 as Q8
    rng = np.random.default_rng(50 + N)
    Wb = _bits(rng, (512, N, 128), 0.02)
    W8, ws = _quant(torch_cuda, Wb, which)
    codes, w_scale = Q8.quant_weight(Wb, which)
    assert np.array_equal(W8.cpu().numpy(), codes)
    assert ws.cpu().numpy()[0] == w_scale


def _check(got, ref, where):
    mx, rel = metrics(got, ref)
    print(where, "max_abs", mx, "rel_l2", rel, flush=True)
    assert mx <= O_MAX_ABS and rel <= O_REL_L2, (where, mx, rel)
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 2.0 ** -12 * np.abs(ref).max()), where


@pytest.mark.parametrize("T,N", [(5, 3), (130, 3), (128, 128)])
def test_absorb_and_up_fp8(torch_cuda, T, N):
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from oracle import bmm8 as Q8
    rng = np.random.default_rng(60 + T + N)
    P = V = 128
    Lkv = 512
    qb = _bits(rng, (T, N, P))
    ob = _bits(rng, (T, N, Lkv), 0.1)
    Wk, Wv = _bits(rng, (Lkv, N, P), 0.02), _bits(rng, (Lkv, N, V), 0.02)
    WK8, wsk = _quant(torch, Wk, "uk")
    WV8, wsv = _quant(torch, Wv, "uv")
    ql = torch.full((T, N, Lkv), float("nan"), dtype=torch.bfloat16, device="cuda")
    o = torch.full((T, N, V), float("nan"), dtype=torch.bfloat16, device="cuda")
    api.mla_absorb_q_fp8(bf16_dev(qb), WK8, wsk, ql)
    api.mla_up_v_fp8(bf16_dev(ob), WV8, wsv, o)
    torch.cuda.synchronize()
    ck, sk = Q8.quant_weight(Wk, "uk")
    cv, sv = Q8.quant_weight(Wv, "uv")
    _check(bf16_host(ql), Q8.absorb_fp8(qb, ck, sk), f"absorb T={T} N={N}")
    _check(bf16_host(o), Q8.up_fp8(ob, cv, sv), f"up T={T} N={N}")
