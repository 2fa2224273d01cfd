"""GPU check of mla_concat_quant_q: fp8 codes bit-exact against the oracle."""
import numpy as np
import pytest

from tests._lib import bf16_dev, ensure_built

pytestmark = pytest.mark.gpu
ensure_built()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    return torch


def _finite_bf16_patterns():
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (allb >> 7) & 0xFF
    return allb[exp != 0xFF]  # drop inf / NaN


@pytest.mark.parametrize("q_scale", [1.0, 0.0123, 5.0 / 448, 3.0])
def test_every_finite_bf16_value_bit_exact(torch_cuda, q_scale):
    from mla_paged_decode_03_amd import api
    from oracle import quant as Q
    torch = torch_cuda
    vals = _finite_bf16_patterns()
    n_rows = -(-len(vals) // 512)
    ql = np.zeros(n_rows * 512, np.uint16)
    ql[:len(vals)] = vals
    ql = ql.reshape(n_rows, 1, 512)
    qp = np.random.default_rng(7).permutation(vals)[: n_rows * 64].reshape(n_rows, 1, 64)
    q8 = torch.zeros((n_rows, 1, 576), dtype=torch.uint8, device="cuda")
    api.mla_concat_quant_q(bf16_dev(ql), bf16_dev(qp), q_scale, q8)
    got = q8.cpu().numpy()
    ref = Q.concat_quant_q(ql, qp, q_scale)
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, (bad[0][:5], got[bad][:5], ref[bad][:5])


def test_strided_views_and_shapes(torch_cuda):
    from mla_paged_decode_03_amd import api
    from oracle import quant as Q
    torch = torch_cuda
    rng = np.random.default_rng(11)
    T, N = 5, 24
    big = (rng.standard_normal((T, N + 3, 512 + 64)) * 4).astype(np.float32)
    bits = (big.view(np.uint32) >> 16).astype(np.uint16)  # truncation to bf16 is fine here
    dev = bf16_dev(bits)
    ql, qp = dev[:, :N, :512], dev[:, :N, 512:]            # head stride 576, token stride 27*576
    q8_big = torch.zeros((T, N + 1, 576 + 16), dtype=torch.uint8, device="cuda")
    q8 = q8_big[:, :N, :576]
    api.mla_concat_quant_q(ql, qp, 0.02, q8)
    ref = Q.concat_quant_q(bits[:, :N, :512], bits[:, :N, 512:], 0.02)
    assert np.array_equal(q8.cpu().numpy(), ref)
    # the padding around the views is untouched
    assert int(q8_big[:, N:, :].to(torch.int32).sum()) == 0 and int(q8_big[:, :, 576:].to(torch.int32).sum()) == 0
