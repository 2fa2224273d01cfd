"""GPU parity of the chunked-prefill path (compute-friendly form) against the oracle.

Pieces: the per-head attention kernel (causal and unmasked, ragged requests, empty
requests and key sets), the context gather (bf16 bit-exact, fp8 within one bf16
rounding of the dequantised value), kv_b_proj, and the whole chunked prefill (several
chunks, requests without context, bf16 and fp8 caches) against the oracle's definition
of the output, with the pipeline's intermediate tensors (dequantised context rows,
k_nope, v) rounded to bf16 as the pages hold them.  Tolerances: the bf16 output bounds of
the decode path (max-abs 1e-2, rel-L2 5e-3) and 1e-3 on the LSE.
"""
import numpy as np
import pytest

from tests._lib import LSE_MAX_ABS, O_MAX_ABS, O_REL_L2, bf16_dev, bf16_host, ensure_built, metrics, u8_dev

pytestmark = pytest.mark.gpu
ensure_built()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    return torch


def _bf16(rng, shape, s=1.0):
    from mla_paged_decode_03_amd.inputs import f32_to_bf16_bits
    return f32_to_bf16_bits((rng.standard_normal(shape) * s).astype(np.float32))


def _check(o, lse, ro, rl, where=""):
    valid = np.isfinite(rl)
    mx, rel = metrics(o, ro)
    dl = np.abs(np.where(valid, lse, 0) - np.where(valid, rl, 0))
    print(where, "max_abs", mx, "rel_l2", rel, "lse", float(dl.max()) if dl.size else 0.0,
          np.unravel_index(np.argmax(dl), dl.shape) if dl.size else None,
          "finite mismatch", int((np.isfinite(lse) != valid).sum()), flush=True)
    assert mx <= O_MAX_ABS and rel <= O_REL_L2, (where, mx, rel)
    assert np.array_equal(np.isfinite(lse), valid), where
    if valid.any():
        assert np.max(np.abs(lse[valid] - rl[valid])) <= LSE_MAX_ABS, where
    assert np.all(o[~valid] == 0), where


@pytest.mark.parametrize("causal,sq,sk", [
    (True, [37, 130, 1, 0, 256], [87, 330, 1, 5, 256]),
    (False, [37, 130, 1, 3, 64], [50, 0, 7, 300, 33]),
    # unmasked launches run the pipelined kernel: odd and even tile counts (3, 5, 32)
    # through its loop and tail steps, query blocks of 256 with ragged ends
    (False, [300, 513, 257], [70, 160, 1000]),
    # causal launches pair query blocks (nqb - 1 - p, p) per workgroup: an odd block
    # count (5: the middle block alone), an even one (4), requests whose high block of a
    # pair is empty, keys beyond the queries (context), and an empty request
    (True, [600, 1100, 257, 0, 900], [700, 1100, 300, 4, 1500]),
    (True, [1024, 513], [1024, 600]),
])
def test_prefill_attention(torch_cuda, causal, sq, sk):
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from oracle import prefill as PF
    from oracle.formats import bf16_to_f64
    rng = np.random.default_rng(31 + causal)
    N, P, R, V = 5, 128, 64, 128
    cq = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(sk)]).astype(np.int32)
    T, S = int(cq[-1]), int(ck[-1])
    qn, qp = _bf16(rng, (T, N, P)), _bf16(rng, (T, N, R))
    kn, kp, v = _bf16(rng, (S, N, P)), _bf16(rng, (S, R)), _bf16(rng, (S, N, V))
    scale = 1.0 / np.sqrt(P + R)
    o = torch.full((T, N, V), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    api.mla_prefill_attention(bf16_dev(qn), bf16_dev(qp), bf16_dev(kn), bf16_dev(kp), bf16_dev(v),
                              torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(), max(sq), causal,
                              scale, o, lse)
    torch.cuda.synchronize()
    go, gl = bf16_host(o), lse.cpu().numpy()
    for b in range(len(sq)):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 == q0:
            continue
        ro, rl = PF.mha(bf16_to_f64(qn[q0:q1]), bf16_to_f64(qp[q0:q1]), bf16_to_f64(kn[k0:k1]),
                        bf16_to_f64(kp[k0:k1]), bf16_to_f64(v[k0:k1]), scale, causal)
        _check(go[q0:q1], gl[q0:q1], ro, rl, f"request {b}")


def test_prefill_attention_dominant_key_exact(torch_cuda):
    """A key whose logit leads every other by far takes all the weight: o equals its
    value row bitwise, in every tile position of the causal window."""
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from mla_paged_decode_03_amd.inputs import f32_to_bf16_bits
    rng = np.random.default_rng(7)
    N, P, R, V, S = 2, 128, 64, 128, 70
    qn = np.zeros((S, N, P), np.uint16)
    kn = np.zeros((S, N, P), np.uint16)
    v = _bf16(rng, (S, N, V))
    # query i points at key (i * 7) % (i + 1), through the rope part only
    kp_f = np.zeros((S, R), np.float32)
    qp_f = np.zeros((S, N, R), np.float32)
    target = np.array([(i * 7) % (i + 1) for i in range(S)])
    for j in range(S):
        kp_f[j, j % R] = 1.0
    for i in range(S):
        qp_f[i, :, target[i] % R] = 3000.0
    # queries whose window holds another key on the target's rope slot would tie: skipped
    ok = np.array([all(j == target[i] or j % R != target[i] % R for j in range(i + 1)) for i in range(S)])
    cq = torch.tensor([0, S], dtype=torch.int32, device="cuda")
    o = torch.empty((S, N, V), dtype=torch.bfloat16, device="cuda")
    api.mla_prefill_attention(bf16_dev(qn), bf16_dev(f32_to_bf16_bits(qp_f)), bf16_dev(kn),
                              bf16_dev(f32_to_bf16_bits(kp_f)), bf16_dev(v), cq, cq, S, True, 1.0, o)
    torch.cuda.synchronize()
    got = o.view(torch.int16).cpu().numpy().view(np.uint16)
    for i in np.nonzero(ok)[0]:
        assert np.array_equal(got[i], v[target[i]]), i


def test_prefill_attention_unmasked_dominant_key_exact(torch_cuda):
    """Unmasked launch (the pipelined kernel): each query has one key whose logit leads
    all others by far, anywhere among 100 keys (4 tiles, the last partial) and across
    two 256-query blocks: o equals that key's value row bitwise."""
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from mla_paged_decode_03_amd.inputs import f32_to_bf16_bits
    rng = np.random.default_rng(11)
    N, P, R, V, Sq, Sk = 3, 128, 64, 128, 300, 100
    v = _bf16(rng, (Sk, N, V))
    kn_f = np.zeros((Sk, N, P), np.float32)
    for j in range(Sk):
        kn_f[j, :, j] = 1.0  # key j: a one in nope dimension j (P = 128 > Sk)
    target = (np.arange(Sq) * 37 + 11) % Sk
    qn_f = np.zeros((Sq, N, P), np.float32)
    for i in range(Sq):
        qn_f[i, :, target[i]] = 3000.0
    qp = np.zeros((Sq, N, R), np.uint16)
    kp = np.zeros((Sk, R), np.uint16)
    cq = torch.tensor([0, Sq], dtype=torch.int32, device="cuda")
    ck = torch.tensor([0, Sk], dtype=torch.int32, device="cuda")
    o = torch.empty((Sq, N, V), dtype=torch.bfloat16, device="cuda")
    api.mla_prefill_attention(bf16_dev(f32_to_bf16_bits(qn_f)), bf16_dev(qp), bf16_dev(f32_to_bf16_bits(kn_f)),
                              bf16_dev(kp), bf16_dev(v), cq, ck, Sq, False, 1.0, o)
    torch.cuda.synchronize()
    got = o.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = [i for i in range(Sq) if not np.array_equal(got[i], v[target[i]])]
    assert not bad, (len(bad), bad[:8])


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_gather_context(torch_cuda, kv_dtype):
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from mla_paged_decode_03_amd import inputs as gen
    from oracle import prefill as PF
    ctx = np.array([100, 0, 257, 16], np.int32)
    w = gen.workload("tiny", B=4, N=1, page_size=16, pool_pages=None, kv_dtype=kv_dtype, seed=41)
    inp = gen.generate(w, seq_lens=ctx)
    mcc, starts, lens, cu = PF.chunk_plan(ctx, 96, 16)
    cache = u8_dev(inp.cache) if kv_dtype == "fp8" else bf16_dev(inp.cache)
    bt = torch.from_numpy(inp.block_table).cuda()
    for i in range(len(starts)):
        tot = int(cu[i, -1])
        okv = torch.empty((max(tot, 1), 512), dtype=torch.bfloat16, device="cuda")
        ope = torch.empty((max(tot, 1), 64), dtype=torch.bfloat16, device="cuda")
        api.mla_gather_context(cache, bt, torch.from_numpy(starts[i].astype(np.int32)).cuda(),
                               torch.from_numpy(cu[i].astype(np.int32)).cuda(), tot, okv, ope,
                               kv_scale=inp.kv_scale)
        torch.cuda.synchronize()
        got = np.concatenate([bf16_host(okv), bf16_host(ope)], axis=1)[:tot]
        ref = np.concatenate([PF.context_rows(inp.cache, kv_dtype, inp.kv_scale, inp.block_table, b,
                                              int(starts[i, b]), int(lens[i, b])) for b in range(len(ctx))])
        if kv_dtype == "bf16":
            assert np.array_equal(got, ref)
        else:  # one rounding of the dequantised value to bf16
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref))


@pytest.mark.parametrize("S,N,P,V,Lkv,row_pad", [
    (300, 3, 128, 128, 512, 0),   # partial tiles in s and n (N*P = 384)
    (1, 1, 8, 16, 512, 0),        # one row, narrow weights
    (600, 16, 128, 128, 512, 64),  # whole n tiles, strided latent rows (row stride 576)
    (257, 2, 64, 40, 96, 0),      # three K chunks of 32, second weight narrower than a tile
    (50, 4, 16, 24, 72, 8),       # Lkv not a multiple of 32: the per-head GEMM
])
def test_kv_b_proj(torch_cuda, S, N, P, V, Lkv, row_pad):
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from oracle import prefill as PF
    from oracle.formats import bf16_to_f64
    rng = np.random.default_rng(43 + S + Lkv)
    kv = _bf16(rng, (S, Lkv + row_pad))
    wk, wv = _bf16(rng, (Lkv, N, P), 0.02), _bf16(rng, (Lkv, N, V), 0.02)
    kn = torch.full((S, N, P), float("nan"), dtype=torch.bfloat16, device="cuda")
    vv = torch.full((S, N, V), float("nan"), dtype=torch.bfloat16, device="cuda")
    api.mla_kv_b_proj(bf16_dev(kv)[:, :Lkv], bf16_dev(wk), bf16_dev(wv), kn, vv)
    torch.cuda.synchronize()
    rk, rv = PF.kv_b_proj(bf16_to_f64(kv[:, :Lkv]), bf16_to_f64(wk), bf16_to_f64(wv))
    for got, ref in ((bf16_host(kn), rk), (bf16_host(vv), rv)):
        mx, rel = metrics(got, ref)
        assert mx <= O_MAX_ABS and rel <= O_REL_L2, (mx, rel)
        # fp32 accumulation, one rounding: within one bf16 step of the exact value
        assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-6)


def test_kv_b_proj_full_size_sampled(torch_cuda):
    """The prefill workload's kv_b_proj shape (8192 latent rows, 128 heads, P = V = 128):
    every output column of 256 sampled rows (spread over all s-tiles) against the oracle."""
    torch = torch_cuda
    from mla_paged_decode_03_amd import api
    from oracle import prefill as PF
    from oracle.formats import bf16_to_f64
    rng = np.random.default_rng(4099)
    S, N, P, V = 8192, 128, 128, 128
    kv = _bf16(rng, (S, 512))
    wk, wv = _bf16(rng, (512, N, P), 0.02), _bf16(rng, (512, N, V), 0.02)
    kn = torch.full((S, N, P), float("nan"), dtype=torch.bfloat16, device="cuda")
    vv = torch.full((S, N, V), float("nan"), dtype=torch.bfloat16, device="cuda")
    api.mla_kv_b_proj(bf16_dev(kv), bf16_dev(wk), bf16_dev(wv), kn, vv)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(S, 256, replace=False))
    rk, rv = PF.kv_b_proj(bf16_to_f64(kv[rows]), bf16_to_f64(wk), bf16_to_f64(wv))
    for got, ref in ((bf16_host(kn[torch.from_numpy(rows).cuda()]), rk),
                     (bf16_host(vv[torch.from_numpy(rows).cuda()]), rv)):
        mx, rel = metrics(got, ref)
        assert mx <= O_MAX_ABS and rel <= O_REL_L2, (mx, rel)
        assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-6)


def _oracle_prefill(inp, requests=None):
    from oracle import prefill as PF
    from oracle.formats import bf16_to_f64
    return PF.chunked_prefill(
        bf16_to_f64(inp.q_nope), bf16_to_f64(inp.q_pe), inp.cu_new, bf16_to_f64(inp.kv_c), bf16_to_f64(inp.k_pe),
        inp.ctx.seq_lens, inp.ctx.cache, inp.ctx.w.kv_dtype, inp.ctx.kv_scale, inp.ctx.block_table,
        bf16_to_f64(inp.W_UK), bf16_to_f64(inp.W_UV), inp.scale, requests=requests, kv_round="bf16")


def run_prefill(torch, inp, workspace_tokens, with_lse=True):
    from mla_paged_decode_03_amd import api
    T, N = inp.T, inp.N
    cache = u8_dev(inp.ctx.cache) if inp.ctx.w.kv_dtype == "fp8" else bf16_dev(inp.ctx.cache)
    ws_bytes = api.mla_chunked_prefill_workspace_size(inp.new_lens, inp.ctx.seq_lens, N, inp.P, inp.V,
                                                     inp.ctx.w.page_size, workspace_tokens)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    o = torch.full((T, N, inp.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
    api.mla_chunked_prefill(bf16_dev(inp.q_nope), bf16_dev(inp.q_pe), bf16_dev(inp.kv_c), bf16_dev(inp.k_pe),
                            inp.new_lens, inp.ctx.seq_lens, cache, torch.from_numpy(inp.ctx.block_table).cuda(),
                            bf16_dev(inp.W_UK), bf16_dev(inp.W_UV), inp.scale, workspace_tokens, o, lse, ws,
                            kv_scale=inp.ctx.kv_scale)
    torch.cuda.synchronize()
    return bf16_host(o), (lse.cpu().numpy() if with_lse else None)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("ctx,new,wt", [
    ([100, 0, 257], [20, 33, 1], 96),      # 6 chunks of 48, a request without context
    ([0, 0], [5, 140], 64),               # no context at all: one causal pass
    ([64, 640], [130, 7], 4096),          # one chunk
])
def test_chunked_prefill(torch_cuda, kv_dtype, ctx, new, wt):
    from mla_paged_decode_03_amd import inputs as gen
    inp = gen.generate_prefill(ctx, new, N=8, page_size=16, kv_dtype=kv_dtype, seed=2100 + len(ctx))
    o, lse = run_prefill(torch_cuda, inp, wt)
    ro, rl = _oracle_prefill(inp)
    _check(o, lse, ro, rl, f"{kv_dtype} ctx={ctx} new={new}")


def test_chunked_prefill_workspace_errors(torch_cuda):
    from mla_paged_decode_03_amd import api
    with pytest.raises(api.MLAError) as e:
        api.mla_chunked_prefill_workspace_size([1, 1, 1], [5, 5, 5], 8, 128, 128, 16, 2)
    assert e.value.status == api.MLA_ERR_WORKSPACE
    from mla_paged_decode_03_amd import inputs as gen
    inp = gen.generate_prefill([40], [3], N=2, page_size=16, seed=5)
    torch = torch_cuda
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    o = torch.empty((3, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.MLAError) as e:
        api.mla_chunked_prefill(bf16_dev(inp.q_nope), bf16_dev(inp.q_pe), bf16_dev(inp.kv_c), bf16_dev(inp.k_pe),
                                inp.new_lens, inp.ctx.seq_lens, bf16_dev(inp.ctx.cache),
                                torch.from_numpy(inp.ctx.block_table).cuda(), bf16_dev(inp.W_UK),
                                bf16_dev(inp.W_UV), inp.scale, 32, o, None, ws)
    assert e.value.status == api.MLA_ERR_WORKSPACE


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_prefill_workload_sampled_parity(torch_cuda, kv_dtype):
    """The full chunked-prefill workload (DSV3 heads, 4 requests of 2048 new tokens after
    6144 tokens of context, 3 context chunks each) in the launch configuration the bench
    times, with a bf16 and an fp8 context cache; sampled (request, head) pairs against the
    oracle, each over all of the request's new tokens (heads are independent: the oracle
    gets that head's slice)."""
    from mla_paged_decode_03_amd import inputs as gen
    from oracle import prefill as PF
    from oracle.formats import bf16_to_f64
    cfg = dict(gen.PREFILL_WORKLOAD)
    wt = cfg.pop("workspace_tokens")
    cfg["kv_dtype"] = kv_dtype
    inp = gen.generate_prefill(**cfg)
    o, lse = run_prefill(torch_cuda, inp, wt)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    qn, qp = bf16_to_f64(inp.q_nope), bf16_to_f64(inp.q_pe)
    kv, kpe = bf16_to_f64(inp.kv_c), bf16_to_f64(inp.k_pe)
    WK, WV = bf16_to_f64(inp.W_UK), bf16_to_f64(inp.W_UV)
    for b, h in ((0, 0), (3, 127), (1, 77)):
        lo, hi = int(inp.cu_new[b]), int(inp.cu_new[b + 1])
        ro, rl = PF.chunked_prefill(qn[:, h:h + 1], qp[:, h:h + 1], inp.cu_new, kv, kpe, inp.ctx.seq_lens,
                                    inp.ctx.cache, inp.ctx.w.kv_dtype, inp.ctx.kv_scale, inp.ctx.block_table,
                                    WK[:, h:h + 1], WV[:, h:h + 1], inp.scale, requests=[b], kv_round="bf16")
        _check(o[lo:hi, h], lse[lo:hi, h], ro[lo:hi, 0], rl[lo:hi, 0], f"request {b} head {h}")


def test_chunked_prefill_without_lse_and_against_unrounded_definition(torch_cuda):
    """lse = None (the running LSE then lives in the workspace) gives the same output as
    with an LSE; and against the unrounded definition (no bf16 rounding of the gathered
    rows, k_nope and v) the output still meets the bf16 bounds, the LSE within 3e-3: the
    bf16 rounding of k_nope moves each logit by about scale * 2^-9 * sum |q||k| (reading of
    the pages' model-dtype intermediates), which the rounded oracle reproduces exactly."""
    from mla_paged_decode_03_amd import inputs as gen
    inp = gen.generate_prefill([100, 0, 257], [20, 33, 1], N=8, page_size=16, kv_dtype="bf16", seed=2103)
    o1, l1 = run_prefill(torch_cuda, inp, 96)
    o2, _ = run_prefill(torch_cuda, inp, 96, with_lse=False)
    assert np.array_equal(o1, o2)
    from oracle import prefill as PF
    from oracle.formats import bf16_to_f64
    ro, rl = PF.chunked_prefill(
        bf16_to_f64(inp.q_nope), bf16_to_f64(inp.q_pe), inp.cu_new, bf16_to_f64(inp.kv_c), bf16_to_f64(inp.k_pe),
        inp.ctx.seq_lens, inp.ctx.cache, inp.ctx.w.kv_dtype, inp.ctx.kv_scale, inp.ctx.block_table,
        bf16_to_f64(inp.W_UK), bf16_to_f64(inp.W_UV), inp.scale)
    mx, rel = metrics(o1, ro)
    dl = float(np.max(np.abs(l1 - rl)))
    print("unrounded definition: max_abs", mx, "rel_l2", rel, "lse", dl, flush=True)
    assert mx <= O_MAX_ABS and rel <= O_REL_L2 and dl <= 3e-3, (mx, rel, dl)
