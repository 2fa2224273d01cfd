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


def test_verify_pipeline_fp8_bmm_end_to_end(torch_cuda):
    """The verify workload at full size (B = 32, Sq = 4, N = 128, P = V = 128, 4096 keys)
    through fp8 absorb -> decode -> fp8 up-projection, as bench.py --workload verify
    --fp8-bmm runs it; 4 sampled requests (16 tokens x 128 heads).

    Stage-wise, each stage gets the GPU's own input and meets the stage bound: the fp8
    products within 2^-7 relative (same quantisation decisions on both sides), the
    latent attention within max-abs 1e-2 / rel-L2 5e-3.  End to end, against the oracle's
    fp8 pipeline from q_nope: the activation quantisation of the up-projection is a step
    function, so an o_latent that differs from the oracle's by the decode's bf16-level
    error (rel-L2 r_d ~ 2e-3) lands on a different e4m3 code with probability about
    |delta| / step; the expected squared change is then about E|delta| * E step, giving
    rel-L2 ~ sqrt(0.8 r_d * 0.09 * 0.8) ~ 0.011 (step about 2^-3.5 of the value); the
    up-projection's random weights carry relative L2 through.  Bound: rel-L2 <= 0.02,
    max-abs <= 1e-2."""
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from mla_paged_decode_03_amd import inputs as gen
    from oracle import attention as A
    from oracle import bmm8 as Q8
    from oracle.formats import bf16_to_f64, to_bf16_bits
    w = gen.workload("verify")
    inp = gen.generate(w)
    T, N, P, V = w.T, w.N, w.P, w.V
    WK8, wsk = _quant(torch, inp.W_UK, "uk")
    WV8, wsv = _quant(torch, inp.W_UV, "uv")
    ck, sk = Q8.quant_weight(inp.W_UK, "uk")
    cv, sv = Q8.quant_weight(inp.W_UV, "uv")
    assert np.array_equal(WK8.cpu().numpy(), ck) and np.array_equal(WV8.cpu().numpy(), cv)
    ql = torch.empty((T, N, 512), dtype=torch.bfloat16, device="cuda")
    api.mla_absorb_q_fp8(bf16_dev(inp.q_nope), WK8, wsk, ql)
    plan = api.mla_decode_plan(inp.seq_lens, w.Sq, N, w.page_size, inp.block_table.shape[1])
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    ol = torch.empty((T, N, 512), dtype=torch.bfloat16, device="cuda")
    api.mla_decode_run(plan, ql, bf16_dev(inp.q_pe), bf16_dev(inp.cache), torch.from_numpy(inp.block_table).cuda(),
                       torch.from_numpy(inp.seq_lens).cuda(), w.scale, inp.kv_scale, ol, None, ws)
    o = torch.empty((T, N, V), dtype=torch.bfloat16, device="cuda")
    api.mla_up_v_fp8(ol, WV8, wsv, o)
    torch.cuda.synchronize()
    plan.destroy()
    reqs = [0, 11, 20, 31]
    rows = np.concatenate([np.arange(b * w.Sq, (b + 1) * w.Sq) for b in reqs])
    ql_bits = ql.view(torch.int16).cpu().numpy().view(np.uint16)
    ol_bits = ol.view(torch.int16).cpu().numpy().view(np.uint16)
    # stage 1: fp8 absorption of the same q_nope
    _check(bf16_host(ql)[rows], Q8.absorb_fp8(inp.q_nope[rows], ck, sk), "absorb (verify, sampled)")
    # stage 2: latent attention fed the GPU's ql_nope
    ro, _ = A.latent_attention(bf16_to_f64(ql_bits), bf16_to_f64(inp.q_pe), inp.cache, w.kv_dtype, inp.kv_scale,
                               inp.block_table, inp.seq_lens, w.Sq, w.scale, requests=reqs)
    ma, rel = metrics(bf16_host(ol)[rows], ro[rows])
    print("latent attention (stage-wise)", ma, rel, flush=True)
    assert ma <= O_MAX_ABS and rel <= O_REL_L2, (ma, rel)
    # stage 3: fp8 up-projection of the GPU's o_latent
    _check(bf16_host(o)[rows], Q8.up_fp8(ol_bits[rows], cv, sv), "up (verify, sampled)")
    # end to end: the oracle's pipeline from q_nope, bf16 between the stages
    rq = bf16_to_f64(to_bf16_bits(Q8.absorb_fp8(inp.q_nope, ck, sk)))
    rl, _ = A.latent_attention(rq, bf16_to_f64(inp.q_pe), inp.cache, w.kv_dtype, inp.kv_scale, inp.block_table,
                               inp.seq_lens, w.Sq, w.scale, requests=reqs)
    ref = Q8.up_fp8(to_bf16_bits(rl[rows]), cv, sv)
    ma, rel = metrics(bf16_host(o)[rows], ref)
    print("end to end vs the oracle's fp8 pipeline: max_abs", ma, "rel_l2", rel, flush=True)
    assert ma <= O_MAX_ABS and rel <= 0.02, (ma, rel)
