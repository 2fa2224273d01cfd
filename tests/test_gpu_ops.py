"""GPU parity of merge_attn_states, the W_UK absorption and the W_UV up-projection."""
import numpy as np
import pytest

from tests._lib import O_MAX_ABS, O_REL_L2, bf16_dev, ensure_built, metrics

pytestmark = pytest.mark.gpu
ensure_built()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    return torch


def _merge_case(seed, T, N, D, dead_frac=0.1):
    from mla_paged_decode_03_amd import inputs as gen
    po = gen.random_f32(seed, 1, (T, N, D))
    so = gen.random_f32(seed, 2, (T, N, D))
    pl = gen.random_f32(seed, 3, (T, N), scale=3.0)
    sl_ = gen.random_f32(seed, 4, (T, N), scale=3.0)
    rng = np.random.default_rng(seed)
    pl[rng.random((T, N)) < dead_frac] = -np.inf
    sl_[rng.random((T, N)) < dead_frac] = -np.inf
    both = rng.random((T, N)) < dead_frac
    pl[both] = -np.inf
    sl_[both] = -np.inf
    return po, pl, so, sl_


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T,N,D", [(3, 16, 512), (5, 7, 128), (1, 128, 576), (2, 3, 1032)])
def test_merge_attn_states(torch_cuda, dtype, T, N, D):
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from mla_paged_decode_03_amd.inputs import f32_to_bf16_bits
    from oracle import attention as A
    from oracle.formats import bf16_to_f64
    po, pl, so, sl_ = _merge_case(T * 100 + N, T, N, D)
    if dtype == "bf16":
        pob, sob = f32_to_bf16_bits(po), f32_to_bf16_bits(so)
        po64, so64 = bf16_to_f64(pob), bf16_to_f64(sob)
        dpo, dso = bf16_dev(pob), bf16_dev(sob)
        out = torch.empty((T, N, D), dtype=torch.bfloat16, device="cuda")
    else:
        po64, so64 = po.astype(np.float64), so.astype(np.float64)
        dpo, dso = torch.from_numpy(po).cuda(), torch.from_numpy(so).cuda()
        out = torch.empty((T, N, D), dtype=torch.float32, device="cuda")
    out_lse = torch.empty((T, N), dtype=torch.float32, device="cuda")
    api.merge_attn_states(out, out_lse, dpo, torch.from_numpy(pl).cuda(), dso,
                          torch.from_numpy(sl_).cuda())
    torch.cuda.synchronize()
    ro, rl = A.merge_states([po64, so64], [pl.astype(np.float64), sl_.astype(np.float64)])
    got = out.float().cpu().numpy()
    if dtype == "fp32":
        np.testing.assert_allclose(got, ro, rtol=2e-5, atol=2e-5)
    else:
        assert np.all(np.abs(got - ro) <= 2.0 ** -8 * np.abs(ro) + 1e-6)
    gl = out_lse.cpu().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(gl)) and np.all(gl[~fin] == -np.inf)
    np.testing.assert_allclose(gl[fin], rl[fin], rtol=0, atol=1e-5)
    assert np.all(got[~fin] == 0)


@pytest.mark.parametrize("T,N,P,Lkv", [(128, 128, 128, 512), (5, 3, 64, 512), (70, 16, 128, 512),
                                       (1, 1, 32, 64), (33, 8, 200, 136)])
def test_absorb_q(torch_cuda, T, N, P, Lkv):
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from mla_paged_decode_03_amd import inputs as gen
    from oracle import attention as A
    from oracle.formats import bf16_to_f64
    q = gen.random_bf16(T + N, 1, (T, N, P))
    W = gen.random_bf16(T + N, 4, (Lkv, N, P), scale=0.02)
    out = torch.full((T, N, Lkv), float("nan"), dtype=torch.bfloat16, device="cuda")
    api.mla_absorb_q(bf16_dev(q), bf16_dev(W), out)
    torch.cuda.synchronize()
    ref = A.absorb(bf16_to_f64(q), bf16_to_f64(W))
    got = out.float().cpu().numpy()
    ma, rel = metrics(got, ref)
    assert ma <= O_MAX_ABS and rel <= O_REL_L2, (ma, rel)


@pytest.mark.parametrize("T,N,Lkv,V", [(128, 128, 512, 128), (5, 3, 512, 64), (70, 16, 512, 128),
                                       (1, 1, 64, 32), (33, 8, 136, 200)])
def test_up_v(torch_cuda, T, N, Lkv, V):
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from mla_paged_decode_03_amd import inputs as gen
    from oracle import attention as A
    from oracle.formats import bf16_to_f64
    x = gen.random_bf16(T + V, 1, (T, N, Lkv), scale=0.1)
    W = gen.random_bf16(T + V, 5, (Lkv, N, V), scale=0.02)
    out = torch.full((T, N, V), float("nan"), dtype=torch.bfloat16, device="cuda")
    api.mla_up_v(bf16_dev(x), bf16_dev(W), out)
    torch.cuda.synchronize()
    ref = A.up_proj(bf16_to_f64(x), bf16_to_f64(W))
    got = out.float().cpu().numpy()
    ma, rel = metrics(got, ref)
    assert ma <= O_MAX_ABS and rel <= O_REL_L2, (ma, rel)


def test_attend_then_reduce_equals_run(torch_cuda):
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from mla_paged_decode_03_amd import inputs as gen
    inp = gen.generate(gen.workload("tiny", B=2, N=64, page_size=64, pool_pages=None, seed=3),
                       seq_lens=np.array([4000, 900], np.int32))
    w = inp.w
    args = (bf16_dev(inp.q), bf16_dev(inp.q_pe), bf16_dev(inp.cache),
            torch.from_numpy(inp.block_table).cuda(), torch.from_numpy(inp.seq_lens).cuda(),
            w.scale, 1.0)
    plan = api.mla_decode_plan(inp.seq_lens, 1, w.N, 64, inp.block_table.shape[1], num_cus=32)
    assert plan.workspace_bytes > 0
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    o1 = torch.empty((2, w.N, 512), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    l1 = torch.empty((2, w.N), dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    api.mla_decode_run(plan, *args, o1, l1, ws)
    api.mla_decode_attend(plan, *args, o2, l2, ws)
    api.mla_decode_reduce(plan, o2, l2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
