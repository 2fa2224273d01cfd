"""Pins of the chunked-prefill oracle (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import prefill as PF

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_chunk_plan_worked_example():
    g = json.load(open(os.path.join(GOLD, "chunk_plan.json")))
    c = g["case"]
    mcc, starts, lens, cu = PF.chunk_plan(c["ctx_lens"], c["workspace_tokens"], c["page_size"])
    assert mcc == g["mcc"]
    assert starts.tolist() == g["starts"]
    assert lens.tolist() == g["lens"]
    assert cu.tolist() == g["cu"]


def test_chunk_plan_rounding_and_requests_without_context():
    # 1000 // 4 = 250, rounded down to the 16-token page: 240
    assert PF.chunk_plan([10, 20, 30, 500], 1000, 16)[0] == 240
    # only requests with context share the workspace
    mcc, starts, lens, cu = PF.chunk_plan([0, 500, 0], 512, 64)
    assert mcc == 512 and lens.tolist() == [[0, 500, 0]] and cu.tolist() == [[0, 0, 500, 500]]
    # a share below one page is kept as is
    assert PF.chunk_plan([100] * 8, 40, 16)[0] == 5
    # no context: no chunks
    assert PF.chunk_plan([0, 0], 256, 16)[0] == 0
    # every context token is covered exactly once
    C = np.array([0, 1, 63, 64, 65, 1000])
    mcc, starts, lens, cu = PF.chunk_plan(C, 256, 16)
    assert (lens.sum(axis=0) == C).all()
    assert ((starts + lens)[lens > 0] <= np.broadcast_to(C, lens.shape)[lens > 0]).all()


def test_kv_b_proj_against_loops():
    rng = np.random.default_rng(5)
    S, Lkv, N, P, V = 3, 6, 2, 4, 5
    kv = rng.standard_normal((S, Lkv))
    Wk = rng.standard_normal((Lkv, N, P))
    Wv = rng.standard_normal((Lkv, N, V))
    k, v = PF.kv_b_proj(kv, Wk, Wv)
    for s in range(S):
        for h in range(N):
            for p in range(P):
                assert abs(k[s, h, p] - sum(kv[s, l] * Wk[l, h, p] for l in range(Lkv))) < 1e-12
            for c in range(V):
                assert abs(v[s, h, c] - sum(kv[s, l] * Wv[l, h, c] for l in range(Lkv))) < 1e-12


def _case(rng, ctx_lens, new_lens, N=2, P=8, R=4, Lkv=16, V=6, ps=4, scale=0.3):
    B = len(ctx_lens)
    cu = np.zeros(B + 1, np.int64)
    cu[1:] = np.cumsum(new_lens)
    T = int(cu[-1])
    pages = [(c + ps - 1) // ps for c in ctx_lens]
    npg = max(1, sum(pages))
    perm = rng.permutation(npg)
    bt = np.full((B, max(1, max(pages))), -1, np.int32)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    f = rng.standard_normal((npg, ps, Lkv + R)).astype(np.float32)
    cache = (f.view(np.uint32) >> 16).astype(np.uint16)  # bf16 bits (truncated: any bits do)
    return dict(q_nope=rng.standard_normal((T, N, P)), q_pe=rng.standard_normal((T, N, R)),
                cu_new=cu, kv_c=rng.standard_normal((T, Lkv)), k_pe=rng.standard_normal((T, R)),
                ctx_lens=np.array(ctx_lens), cache_bits=cache, cache_dtype="bf16", kv_scale=1.0,
                block_table=bt, W_UK=rng.standard_normal((Lkv, N, P)) * 0.3,
                W_UV=rng.standard_normal((Lkv, N, V)), scale=scale)


@pytest.mark.parametrize("seed", range(3))
def test_definition_equals_the_chunk_loop(seed):
    """The docstring's algorithm (causal suffix, context chunks each merged in, then the
    prefix/suffix merge) reproduces the definition."""
    rng = np.random.default_rng(100 + seed)
    ctx_lens, new_lens = [9, 0, 23], [5, 3, 1]
    c = _case(rng, ctx_lens, new_lens)
    o_ref, lse_ref = PF.chunked_prefill(**c)
    Lkv = c["W_UK"].shape[0]
    mcc, starts, lens, cu = PF.chunk_plan(ctx_lens, 12, 4)
    assert mcc == 4 and len(starts) == 6
    for b in range(len(ctx_lens)):
        lo, hi = c["cu_new"][b], c["cu_new"][b + 1]
        kn, v = PF.kv_b_proj(c["kv_c"][lo:hi], c["W_UK"], c["W_UV"])
        suf_o, suf_l = PF.mha(c["q_nope"][lo:hi], c["q_pe"][lo:hi], kn, c["k_pe"][lo:hi], v,
                              c["scale"], causal=True)
        pre = None
        for i in range(len(starts)):
            rows = PF.context_rows(c["cache_bits"], "bf16", 1.0, c["block_table"], b,
                                   int(starts[i, b]), int(lens[i, b]))
            kn, v = PF.kv_b_proj(rows[:, :Lkv], c["W_UK"], c["W_UV"])
            co, cl = PF.mha(c["q_nope"][lo:hi], c["q_pe"][lo:hi], kn, rows[:, Lkv:], v, c["scale"],
                            causal=False)
            pre = (co, cl) if pre is None else A.merge_states([pre[0], co], [pre[1], cl])
        o, lse = A.merge_states([pre[0], suf_o], [pre[1], suf_l])
        np.testing.assert_allclose(o, o_ref[lo:hi], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref[lo:hi], rtol=1e-10, atol=1e-12)


def test_definition_equals_the_absorbed_latent_path():
    """With the new rows appended to the context in the cache, the absorbed MQA decode of
    the same queries (Sq = new tokens per request, causal verify window), up-projected with
    W_UV, is the same attention (docstring: the two approaches compute the same result)."""
    rng = np.random.default_rng(7)
    N, P, R, Lkv, V, ps, S = 3, 8, 4, 16, 6, 4, 3
    ctx_lens = [10, 4]
    c = _case(rng, ctx_lens, [S, S], N=N, P=P, R=R, Lkv=Lkv, V=V, ps=ps)
    bits = lambda x: (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    # make every value exactly representable in bf16 so both paths read the same numbers
    from oracle.formats import bf16_to_f64
    c["kv_c"] = bf16_to_f64(bits(c["kv_c"]))
    c["k_pe"] = bf16_to_f64(bits(c["k_pe"]))
    o_ref, lse_ref = PF.chunked_prefill(**c)
    # cache holding context + new rows for each request
    L = [C + S for C in ctx_lens]
    pages = [(x + ps - 1) // ps for x in L]
    cache = np.zeros((sum(pages), ps, Lkv + R), np.uint16)
    bt = np.full((2, max(pages)), -1, np.int32)
    off = 0
    for b in range(2):
        bt[b, :pages[b]] = np.arange(off, off + pages[b])[::-1]
        off += pages[b]
        ctx = PF.context_rows(c["cache_bits"], "bf16", 1.0, c["block_table"], b, 0, ctx_lens[b])
        lo = c["cu_new"][b]
        rows = np.concatenate([ctx, np.concatenate([c["kv_c"][lo:lo + S], c["k_pe"][lo:lo + S]], 1)])
        for j in range(L[b]):
            cache[bt[b, j // ps], j % ps] = bits(rows[j])
    ql = A.absorb(c["q_nope"], c["W_UK"])
    o_lat, lse = A.latent_attention(ql, c["q_pe"], cache, "bf16", 1.0, bt, np.array(L), S, c["scale"],
                                    Lkv=Lkv)
    np.testing.assert_allclose(A.up_proj(o_lat, c["W_UV"]), o_ref, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-10, atol=1e-12)


def test_zero_queries_average_the_visible_values():
    """q = 0: every visible key has logit 0, so o = mean of the visible values and
    lse = ln(count); new token i of a request with C context tokens sees C + i + 1 keys."""
    rng = np.random.default_rng(11)
    ctx_lens, new_lens = [5, 0], [4, 2]
    c = _case(rng, ctx_lens, new_lens)
    c["q_nope"][:] = 0
    c["q_pe"][:] = 0
    o, lse = PF.chunked_prefill(**c)
    Lkv = c["W_UK"].shape[0]
    for b, C in enumerate(ctx_lens):
        lo = c["cu_new"][b]
        ctx = PF.context_rows(c["cache_bits"], "bf16", 1.0, c["block_table"], b, 0, C)
        lat = np.concatenate([ctx[:, :Lkv], c["kv_c"][lo:lo + new_lens[b]]])
        vals = lat @ c["W_UV"].reshape(Lkv, -1)
        for i in range(new_lens[b]):
            n = C + i + 1
            np.testing.assert_allclose(o[lo + i].reshape(-1), vals[:n].mean(axis=0), rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse[lo + i], math.log(n), rtol=1e-12)


def test_brute_force_tiny():
    rng = np.random.default_rng(13)
    c = _case(rng, [3], [2], N=2, P=3, R=2, Lkv=4, V=2, ps=2)
    o, lse = PF.chunked_prefill(**c)
    ctx = PF.context_rows(c["cache_bits"], "bf16", 1.0, c["block_table"], 0, 0, 3)
    lat = np.concatenate([ctx[:, :4], c["kv_c"]])
    pe = np.concatenate([ctx[:, 4:], c["k_pe"]])
    for t in range(2):
        for h in range(2):
            keys, vals = [], []
            for j in range(3 + t + 1):
                kn = [sum(lat[j, l] * c["W_UK"][l, h, p] for l in range(4)) for p in range(3)]
                keys.append(kn + list(pe[j]))
                vals.append([sum(lat[j, l] * c["W_UV"][l, h, x] for l in range(4)) for x in range(2)])
            q = list(c["q_nope"][t, h]) + list(c["q_pe"][t, h])
            ob, lb = A.attention_brute([q], keys, vals, c["scale"])
            np.testing.assert_allclose(o[t, h], ob[0], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse[t, h], lb[0], rtol=1e-12)


def test_fp8_context_is_dequantised_with_the_scale():
    """An fp8 cache holds e4m3fn codes; the context rows are code value * kv_scale."""
    import torch
    rng = np.random.default_rng(17)
    codes = rng.integers(0, 256, size=(2, 4, 20), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0  # no NaN codes
    bt = np.array([[1, 0]], np.int32)
    rows = PF.context_rows(codes, "fp8", 0.5, bt, 0, 2, 5)
    ref = torch.from_numpy(codes.reshape(-1, 20)).view(torch.float8_e4m3fn).double().numpy() * 0.5
    flat_rows = [1 * 4 + 2, 1 * 4 + 3, 0 * 4 + 0, 0 * 4 + 1, 0 * 4 + 2]
    np.testing.assert_array_equal(rows, ref[flat_rows])


def test_rounded_pipeline_is_exact_when_nothing_rounds():
    """kv_round="bf16" only rounds the intermediate tensors: with W_UK / W_UV selecting
    single latent columns (k_nope and v are copies of bf16 cache values) nothing changes."""
    rng = np.random.default_rng(23)
    ctx_lens, new_lens = [9, 0, 23], [5, 3, 1]
    c = _case(rng, ctx_lens, new_lens)
    Lkv, N, P = c["W_UK"].shape
    V = c["W_UV"].shape[2]
    from oracle.formats import round_to_bf16
    c["kv_c"] = round_to_bf16(c["kv_c"])
    wk = np.zeros((Lkv, N, P))
    wv = np.zeros((Lkv, N, V))
    for h in range(N):
        for p in range(P):
            wk[(3 * h + p) % Lkv, h, p] = 1.0
        for q in range(V):
            wv[(5 * h + q) % Lkv, h, q] = 1.0
    c["W_UK"], c["W_UV"] = wk, wv
    o0, l0 = PF.chunked_prefill(**c)
    o1, l1 = PF.chunked_prefill(**c, kv_round="bf16")
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # and with general weights the rounded pipeline moves the output by about a bf16 step
    c2 = _case(np.random.default_rng(24), ctx_lens, new_lens)
    o0, _ = PF.chunked_prefill(**c2)
    o1, _ = PF.chunked_prefill(**c2, kv_round="bf16")
    assert 0 < np.max(np.abs(o1 - o0)) < 2.0 ** -5 * max(1.0, np.max(np.abs(o0)))

