"""GPU check of mla_concat_and_cache: the cache bytes bit-exact against the oracle, and a
decode over rows written by it."""
import numpy as np
import pytest

from tests._lib import bf16_dev, bf16_host, ensure_built, metrics, O_MAX_ABS, O_REL_L2

pytestmark = pytest.mark.gpu
ensure_built()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    return torch


def _tokens(rng, T, scale=2.0):
    x = (rng.standard_normal((T, 576)) * scale).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    return np.ascontiguousarray(bits[:, :512]), np.ascontiguousarray(bits[:, 512:])


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
@pytest.mark.parametrize("ps,pages,T", [(1, 40, 33), (16, 9, 100), (64, 4, 200)])
def test_cache_bytes_bit_exact(torch_cuda, dt, ps, pages, T):
    import torch
    from mla_paged_decode_03_amd import api
    from oracle import cache as CW
    rng = np.random.default_rng(ps * 1000 + T)
    kv, pe = _tokens(rng, T)
    slots = rng.permutation(pages * ps)[:T].astype(np.int64)
    slots[rng.random(T) < 0.1] = -1                      # padding tokens
    k_scale = 0.011
    if dt == "bf16":
        init = rng.integers(0, 1 << 16, size=(pages, ps, 576), dtype=np.uint16) & 0x3FFF
        cache = bf16_dev(init)
    else:
        init = rng.integers(0, 0x7E, size=(pages, ps, 576), dtype=np.uint8)
        cache = torch.from_numpy(init).cuda()
    api.mla_concat_and_cache(bf16_dev(kv), bf16_dev(pe), torch.from_numpy(slots).cuda(), cache, k_scale)
    torch.cuda.synchronize()
    got = cache.view(torch.int16).cpu().numpy().view(np.uint16) if dt == "bf16" else cache.cpu().numpy()
    ref = CW.concat_and_cache(kv, pe, slots, init, dt, k_scale)
    assert np.array_equal(got, ref)


def test_strided_token_rows(torch_cuda):
    import torch
    from mla_paged_decode_03_amd import api
    from oracle import cache as CW
    rng = np.random.default_rng(3)
    T = 20
    x = bf16_dev(np.ascontiguousarray(np.concatenate(_tokens(rng, T), axis=1)))  # [T, 576]
    kv, pe = x[:, :512], x[:, 512:]                                               # token stride 576
    init = np.zeros((2, 16, 576), np.uint16)
    cache = bf16_dev(init)
    slots = np.arange(T, dtype=np.int64)[::-1].copy()
    api.mla_concat_and_cache(kv, pe, torch.from_numpy(slots).cuda(), cache)
    bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = CW.concat_and_cache(bits[:, :512], bits[:, 512:], slots, init, "bf16")
    assert np.array_equal(cache.view(torch.int16).cpu().numpy().view(np.uint16), ref)


def test_decode_over_written_rows(torch_cuda):
    """Rows written by the library into an fp8 cache, then decoded: parity with the oracle
    over the oracle's own write of the same rows."""
    import torch
    from mla_paged_decode_03_amd import api
    from oracle import attention as A
    from oracle import cache as CW
    from oracle.formats import bf16_to_f64
    rng = np.random.default_rng(4)
    ps, pages, N = 64, 12, 128
    perm = rng.permutation(pages).astype(np.int32)
    bt = np.full((2, 11), -1, np.int32)
    bt[0, :11] = perm[:11]   # request 0: 700 keys on 11 pages
    bt[1, :1] = perm[11:12]  # request 1: 60 keys on the 12th
    lens = np.array([700, 60], np.int32)
    slots = np.concatenate([[bt[b, j // ps] * ps + j % ps for j in range(lens[b])] for b in range(2)]).astype(np.int64)
    kv, pe = _tokens(rng, len(slots), scale=1.0)
    k_scale = 4.5 / 448
    cache = torch.zeros((pages, ps, 576), dtype=torch.uint8, device="cuda")
    api.mla_concat_and_cache(bf16_dev(kv), bf16_dev(pe), torch.from_numpy(slots).cuda(), cache, k_scale)
    ref_cache = CW.concat_and_cache(kv, pe, slots, np.zeros((pages, ps, 576), np.uint8), "fp8", k_scale)
    assert np.array_equal(cache.cpu().numpy(), ref_cache)
    q = (rng.standard_normal((2, N, 576)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ql, qpe = np.ascontiguousarray(q[..., :512]), np.ascontiguousarray(q[..., 512:])
    plan = api.mla_decode_plan(lens, 1, N, ps, 11, api.MLA_DT_FP8_E4M3FN)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    o = torch.empty((2, N, 512), dtype=torch.bfloat16, device="cuda")
    scale = 1 / np.sqrt(192)
    api.mla_decode_run(plan, bf16_dev(ql), bf16_dev(qpe), cache, torch.from_numpy(bt).cuda(),
                       torch.from_numpy(lens).cuda(), scale, k_scale, o, None, ws)
    torch.cuda.synchronize()
    ro, _ = A.latent_attention(bf16_to_f64(ql), bf16_to_f64(qpe), ref_cache, "fp8", k_scale, bt, lens, 1, scale)
    ma, rel = metrics(bf16_host(o), ro)
    assert ma <= O_MAX_ABS and rel <= O_REL_L2, (ma, rel)
