"""The allocation-free decode entry point (mla_decode_run_noalloc) against mla_decode_run.

Both run the same kernels on the same plan; the only difference is where the split
partial states live (the library's static device scratch instead of a caller's
workspace), so the outputs must be bitwise equal.  Two calls in a row, the second on a
smaller problem, check that the scratch's leftover contents from the first call do not
leak into the second.
"""
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


def _case(seq_lens, N, Sq, ps, seed):
    from mla_paged_decode_03_amd import inputs as gen
    w = gen.workload("tiny", B=len(seq_lens), N=N, Sq=Sq, page_size=ps, pool_pages=None, seed=seed)
    return gen.generate(w, seq_lens=np.array(seq_lens, np.int32))


def _run_both(torch, inp, num_cus):
    from mla_paged_decode_03_amd import api
    w = inp.w
    T, N = w.T, w.N
    q, qpe, cache = bf16_dev(inp.q), bf16_dev(inp.q_pe), bf16_dev(inp.cache)
    bt = torch.from_numpy(inp.block_table).cuda()
    sl = torch.from_numpy(inp.seq_lens).cuda()
    plan = api.mla_decode_plan(inp.seq_lens, w.Sq, N, w.page_size, inp.block_table.shape[1], num_cus=num_cus)
    assert plan.workspace_bytes > 0  # the case is split: the scratch is used
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    o_ref = torch.full((T, N, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    l_ref = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    api.mla_decode_run(plan, q, qpe, cache, bt, sl, w.scale, inp.kv_scale, o_ref, l_ref, ws)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    api.mla_decode_run_noalloc(plan, q, qpe, cache, bt, sl, w.scale, inp.kv_scale, o, lse)
    torch.cuda.synchronize()
    plan.destroy()
    return o.cpu(), lse.cpu(), o_ref.cpu(), l_ref.cpu()


def test_noalloc_matches_run_twice_second_smaller(torch_cuda):
    torch = torch_cuda
    big = _case([5000, 3100, 77, 2600], N=128, Sq=1, ps=64, seed=41)
    small = _case([900, 40], N=16, Sq=2, ps=16, seed=43)
    for inp, cus in ((big, 40), (small, 6)):
        print("noalloc case", inp.w.B, inp.w.N, inp.w.Sq, list(inp.seq_lens), flush=True)
        o, lse, o_ref, l_ref = _run_both(torch, inp, cus)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse, l_ref)
        assert torch.isfinite(o.float()).all()


def test_noalloc_rejects_plans_beyond_the_scratch(torch_cuda):
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    # 8 head groups of 128 rows and 100 partial slots: about 105 MB of workspace
    L = np.array([100000, 100000], np.int32)
    plan = api.mla_decode_plan(L, 8, 128, 64, (100000 + 63) // 64, num_cus=800)  # host-side rejection below
    assert plan.workspace_bytes > 64 << 20
    inp = _case([64, 64], N=128, Sq=8, ps=64, seed=47)  # tensors only need the right types
    q, qpe, cache = bf16_dev(inp.q), bf16_dev(inp.q_pe), bf16_dev(inp.cache)
    pages = (100000 + 63) // 64
    bt = torch.zeros((2, pages), dtype=torch.int32, device="cuda")
    sl = torch.from_numpy(L).cuda()
    o = torch.empty((16, 128, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.MLAError) as e:
        api.mla_decode_run_noalloc(plan, q, qpe, cache, bt, sl, 0.1, 1.0, o)
    assert e.value.status == api.MLA_ERR_WORKSPACE and "static scratch" in str(e.value)
    plan.destroy()
