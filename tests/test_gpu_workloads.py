"""The five workloads at full size on the GPU, in the launch configuration bench.py times,
with sampled requests compared element by element against the fp64 oracle."""
import numpy as np
import pytest

from tests._lib import (LSE_MAX_ABS, O_MAX_ABS, O_REL_L2, bf16_dev, bf16_host, ensure_built,
                        metrics, u8_dev)

pytestmark = pytest.mark.gpu
ensure_built()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    return torch


def _sample(seq_lens):
    L = np.asarray(seq_lens)
    return sorted({0, int(np.argmax(L)), int(np.argmin(L)), len(L) // 2})


@pytest.mark.parametrize("name", ["tiny", "dsv3", "longtail", "verify", "fp8"])
def test_workload_sampled_parity(torch_cuda, name):
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from mla_paged_decode_03_amd import inputs as gen
    from oracle import attention as A
    from oracle.formats import bf16_to_f64
    w = gen.workload(name)
    inp = gen.generate(w)
    dev = "cuda"
    T, N = w.T, w.N
    q_pe = bf16_dev(inp.q_pe)
    cache = bf16_dev(inp.cache) if w.kv_dtype == "bf16" else u8_dev(inp.cache)
    dt = api.MLA_DT_BF16 if w.kv_dtype == "bf16" else api.MLA_DT_FP8_E4M3FN
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.seq_lens).to(dev)
    o = torch.empty((T, N, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, N), dtype=torch.float32, device=dev)
    plan = api.mla_decode_plan(inp.seq_lens, w.Sq, N, w.page_size, inp.block_table.shape[1], dt)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    if w.absorb:
        ql = torch.empty((T, N, 512), dtype=torch.bfloat16, device=dev)
        api.mla_absorb_q(bf16_dev(inp.q_nope), bf16_dev(inp.W_UK), ql)
    else:
        ql = bf16_dev(inp.q)
    api.mla_decode_run(plan, ql, q_pe, cache, bt, sl, w.scale, inp.kv_scale, o, lse, ws)
    if w.absorb:
        out = torch.empty((T, N, w.V), dtype=torch.bfloat16, device=dev)
        api.mla_up_v(o, bf16_dev(inp.W_UV), out)
    torch.cuda.synchronize()
    reqs = _sample(inp.seq_lens)
    rows = np.concatenate([np.arange(b * w.Sq, (b + 1) * w.Sq) for b in reqs])
    if w.absorb:
        # stage-wise: the oracle attention is fed the GPU's bf16 ql_nope; end to end: fp64 absorb
        ql_gpu = ql.float().cpu().numpy().astype(np.float64)
        ro, rl = A.latent_attention(ql_gpu, bf16_to_f64(inp.q_pe), inp.cache, w.kv_dtype,
                                    inp.kv_scale, inp.block_table, inp.seq_lens, w.Sq, w.scale,
                                    requests=reqs)
        got = bf16_host(o)[rows]
        ma, rel = metrics(got, ro[rows])
        assert ma <= O_MAX_ABS and rel <= O_REL_L2, ("stage-wise latent", ma, rel)
        rq = A.absorb(bf16_to_f64(inp.q_nope[rows]), bf16_to_f64(inp.W_UK))
        qfull = np.zeros((T, N, 512))
        qfull[rows] = rq
        ro2, _ = A.latent_attention(qfull, bf16_to_f64(inp.q_pe), inp.cache, w.kv_dtype,
                                    inp.kv_scale, inp.block_table, inp.seq_lens, w.Sq, w.scale,
                                    requests=reqs)
        ref = A.up_proj(ro2[rows], bf16_to_f64(inp.W_UV))
        ma, rel = metrics(bf16_host(out)[rows], ref)
        assert ma <= O_MAX_ABS and rel <= O_REL_L2, ("end to end", ma, rel)
    else:
        ro, rl = A.latent_attention(bf16_to_f64(inp.q), bf16_to_f64(inp.q_pe), inp.cache,
                                    w.kv_dtype, inp.kv_scale, inp.block_table, inp.seq_lens, w.Sq,
                                    w.scale, requests=reqs)
        got = bf16_host(o)[rows]
        ma, rel = metrics(got, ro[rows])
        assert ma <= O_MAX_ABS and rel <= O_REL_L2, (ma, rel)
        gl = lse.cpu().numpy()[rows]
        assert np.max(np.abs(gl - rl[rows])) <= LSE_MAX_ABS
    # every output row is finite (rows not sampled included)
    assert torch.isfinite(o.float()).all()
    plan.destroy()


def test_fp8_workload_with_fp8_query_sampled_parity(torch_cuda):
    """The fp8 workload at full size on the fp8-query path (bench.py --q8): the query is
    quantised on the GPU with the static scale max|q| / 448; sampled requests are compared
    with the oracle fed the same quantised query."""
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from mla_paged_decode_03_amd import inputs as gen
    from oracle import attention as A
    from oracle import quant as Q
    from oracle.formats import E4M3FN_TABLE, bf16_to_f64
    w = gen.workload("fp8")
    inp = gen.generate(w)
    T, N = w.T, w.N
    q_scale = float(np.float32(max(np.abs(bf16_to_f64(inp.q)).max(), np.abs(bf16_to_f64(inp.q_pe)).max()) / 448))
    q8 = torch.empty((T, N, 576), dtype=torch.uint8, device="cuda")
    api.mla_concat_quant_q(bf16_dev(inp.q), bf16_dev(inp.q_pe), q_scale, q8)
    cache = u8_dev(inp.cache)
    bt = torch.from_numpy(inp.block_table).cuda()
    sl = torch.from_numpy(inp.seq_lens).cuda()
    o = torch.empty((T, N, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, N), dtype=torch.float32, device="cuda")
    plan = api.mla_decode_plan(inp.seq_lens, w.Sq, N, w.page_size, inp.block_table.shape[1],
                               api.MLA_DT_FP8_E4M3FN)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    api.mla_decode_run_q8(plan, q8, q_scale, cache, bt, sl, w.scale, inp.kv_scale, o, lse, ws)
    torch.cuda.synchronize()
    reqs = _sample(inp.seq_lens)
    rq8 = Q.concat_quant_q(inp.q[reqs], inp.q_pe[reqs], q_scale)
    assert np.array_equal(q8.cpu().numpy()[reqs], rq8)
    ql = np.zeros((T, N, 512))
    qpe = np.zeros((T, N, 64))
    ql[reqs] = E4M3FN_TABLE[rq8[..., :512]] * q_scale
    qpe[reqs] = E4M3FN_TABLE[rq8[..., 512:]] * q_scale
    ro, rl = A.latent_attention(ql, qpe, inp.cache, "fp8", inp.kv_scale, inp.block_table, inp.seq_lens,
                                w.Sq, w.scale, requests=reqs)
    ma, rel = metrics(bf16_host(o)[reqs], ro[reqs])
    assert ma <= O_MAX_ABS and rel <= O_REL_L2, (ma, rel)
    assert np.max(np.abs(lse.cpu().numpy()[reqs] - rl[reqs])) <= LSE_MAX_ABS
    assert torch.isfinite(o.float()).all()
    plan.destroy()
