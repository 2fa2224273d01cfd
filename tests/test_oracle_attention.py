"""Pins of the fp64 attention oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code path: scalar brute
force, torch's scaled_dot_product_attention (the routine the docstring's
pseudo-code calls), the compute-friendly MHA path, closed forms and
invariances.  A dropped term, a wrong sign, a transposed operand or an
off-by-one in the paging or the causal window fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.formats import bf16_to_f64

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(seed, B, N, Lkv, R, ps, lens, Sq=1, pool_extra=2):
    """f64 values stored as bf16 bits so that the oracle's decoding path is used."""
    rng = np.random.default_rng(seed)
    pages = [(L + ps - 1) // ps for L in lens]
    num_pages = sum(pages) + pool_extra
    perm = rng.permutation(num_pages)
    bt = np.full((B, max(1, max(pages))), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    pool = rng.standard_normal((num_pages, ps, Lkv + R)).astype(np.float32)
    bits = (pool.view(np.uint32) >> 16).astype(np.uint16)  # truncate: any bf16 values will do
    T = B * Sq
    ql = rng.standard_normal((T, N, Lkv))
    qpe = rng.standard_normal((T, N, R))
    return ql, qpe, bits, bt, np.array(lens, dtype=np.int32)


def _keys_for(bits, bt, b, n, ps, Lkv):
    flat = bf16_to_f64(bits.reshape(-1, bits.shape[2]))
    rows = [int(bt[b, j // ps]) * ps + j % ps for j in range(n)]
    kv = flat[rows]
    return kv[:, :Lkv], kv[:, Lkv:]


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    B, N, Lkv, R, ps = 2, 3, 8, 4, 3
    lens = [int(x) for x in rng.integers(1, 8, size=B)]
    ql, qpe, bits, bt, L = _rand_case(seed, B, N, Lkv, R, ps, lens)
    scale = 0.37
    o, lse = A.latent_attention(ql, qpe, bits, "bf16", 1.0, bt, L, 1, scale, Lkv=Lkv)
    for b in range(B):
        kc, kr = _keys_for(bits, bt, b, lens[b], ps, Lkv)
        keys = np.concatenate([kc, kr], 1).tolist()
        qrows = np.concatenate([ql[b], qpe[b]], 1).tolist()
        ob, lb = A.attention_brute(qrows, keys, kc.tolist(), scale)
        np.testing.assert_allclose(o[b], ob, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[b], lb, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("Sq", [1, 3])
def test_matches_torch_sdpa_fp64(Sq):
    B, N, Lkv, R, ps = 2, 4, 16, 8, 4
    lens = [9, 14]
    ql, qpe, bits, bt, L = _rand_case(11, B, N, Lkv, R, ps, lens, Sq=Sq)
    scale = 1 / math.sqrt(24)
    o, lse = A.latent_attention(ql, qpe, bits, "bf16", 1.0, bt, L, Sq, scale, Lkv=Lkv)
    for b in range(B):
        kc, kr = _keys_for(bits, bt, b, lens[b], ps, Lkv)
        q = torch.from_numpy(np.concatenate([ql[b * Sq:(b + 1) * Sq], qpe[b * Sq:(b + 1) * Sq]], 2))
        q = q.permute(1, 0, 2)  # [N, Sq, D]
        k = torch.from_numpy(np.concatenate([kc, kr], 1))[None].expand(N, -1, -1)
        v = torch.from_numpy(kc)[None].expand(N, -1, -1)
        n_vis = [A.visible_keys(lens[b], Sq, t) for t in range(Sq)]
        mask = torch.tensor([[j < n_vis[t] for j in range(lens[b])] for t in range(Sq)])
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(o[b * Sq:(b + 1) * Sq], ref.permute(1, 0, 2).numpy(), rtol=1e-12,
                                   atol=1e-13)
        s = scale * torch.einsum("nqd,nkd->nqk", q, k)
        s = s.masked_fill(~mask[None], float("-inf"))
        ref_lse = torch.logsumexp(s, dim=-1).permute(1, 0).numpy()
        np.testing.assert_allclose(lse[b * Sq:(b + 1) * Sq], ref_lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Sq", [1, 2, 4])
def test_absorbed_equals_compute_friendly(Sq):
    """The two computation paths of the mla/common.py docstring give the same attention."""
    rng = np.random.default_rng(5 + Sq)
    N, P, R, V, Lkv, L = 3, 8, 4, 6, 16, 11
    q_nope = rng.standard_normal((Sq, N, P))
    q_pe = rng.standard_normal((Sq, N, R))
    kv_c = rng.standard_normal((L, Lkv))
    k_pe = rng.standard_normal((L, R))
    W_UK = 0.3 * rng.standard_normal((Lkv, N, P))
    W_UV = 0.3 * rng.standard_normal((Lkv, N, V))
    scale = 1 / math.sqrt(P + R)
    # absorbed: ql = q_nope . W_UK ; latent attention over [kv_c | k_pe] ; up-project with W_UV
    ql = A.absorb(q_nope, W_UK)
    ps = 4
    npg = (L + ps - 1) // ps
    pool = np.zeros((npg, ps, Lkv + R), dtype=np.float32)
    flat = np.concatenate([kv_c, k_pe], 1)
    pool.reshape(-1, Lkv + R)[:L] = flat
    # store exactly: bf16 bits cannot hold arbitrary f64, so compare through a pool whose
    # values are exact bf16 numbers
    bits = (pool.view(np.uint32) >> 16).astype(np.uint16)
    exact = bf16_to_f64(bits).reshape(-1, Lkv + R)[:L]
    kv_c2, k_pe2 = exact[:, :Lkv], exact[:, Lkv:]
    o_mha, lse_mha = A.mha_compute_friendly(q_nope, q_pe, kv_c2, k_pe2, W_UK, W_UV, scale, Sq)
    bt = np.arange(npg, dtype=np.int32)[None]
    o_lat, lse = A.latent_attention(ql, q_pe, bits, "bf16", 1.0, bt, np.array([L]), Sq, scale, Lkv=Lkv)
    o = A.up_proj(o_lat, W_UV)
    np.testing.assert_allclose(o, o_mha, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse_mha, rtol=1e-10, atol=1e-12)


def test_absorb_and_up_against_loops():
    rng = np.random.default_rng(3)
    T, N, P, Lkv, V = 2, 3, 5, 7, 4
    q = rng.standard_normal((T, N, P))
    Wk = rng.standard_normal((Lkv, N, P))
    Wv = rng.standard_normal((Lkv, N, V))
    ql = A.absorb(q, Wk)
    for t in range(T):
        for h in range(N):
            for l in range(Lkv):
                assert abs(ql[t, h, l] - sum(q[t, h, p] * Wk[l, h, p] for p in range(P))) < 1e-12
    o = A.up_proj(ql, Wv)
    for t in range(T):
        for h in range(N):
            for v in range(V):
                assert abs(o[t, h, v] - sum(ql[t, h, l] * Wv[l, h, v] for l in range(Lkv))) < 1e-11


@pytest.mark.parametrize("seed", range(4))
def test_split_merge_exactness(seed):
    rng = np.random.default_rng(40 + seed)
    M, D, Dv, n = 5, 12, 9, 40
    q = rng.standard_normal((M, D))
    k = rng.standard_normal((n, D))
    v = rng.standard_normal((n, Dv))
    o_ref, l_ref = A.attend(q, k, v, 0.5)
    cuts = sorted(set(rng.integers(0, n + 1, size=4).tolist()) | {0, n})
    parts = [A.attend(q, k[a:b], v[a:b], 0.5) for a, b in zip(cuts[:-1], cuts[1:])]
    parts.append(A.attend(q, k[:0], v[:0], 0.5))  # an empty part: lse = -inf, o = 0
    o, l = A.merge_states([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, rtol=1e-12, atol=1e-13)
    # two-way merge in either order is the same
    a, b = A.attend(q, k[:17], v[:17], 0.5), A.attend(q, k[17:], v[17:], 0.5)
    o1, l1 = A.merge_states([a[0], b[0]], [a[1], b[1]])
    o2, l2 = A.merge_states([b[0], a[0]], [b[1], a[1]])
    np.testing.assert_allclose(o1, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-14, atol=1e-15)


def test_merge_of_empty_states():
    o, l = A.merge_states([np.full((2, 3), 5.0), np.full((2, 3), 7.0)], [np.full(2, -np.inf)] * 2)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    # one empty side leaves the other unchanged
    o, l = A.merge_states([np.full((1, 3), 5.0), np.full((1, 3), 7.0)], [np.array([-np.inf]), np.array([1.5])])
    assert np.all(o == 7.0) and l[0] == 1.5


def test_head_independence_with_tiled_padding():
    """Padding heads by tiling q (rocm_aiter_mla page, AiterMLAHelper.get_mla_padded_q) cannot
    change the real heads: each head's output depends only on its own query row and the
    latent cache, so extra query rows leave the others untouched."""
    B, N, Lkv, R, ps = 2, 12, 16, 8, 4
    ql, qpe, bits, bt, L = _rand_case(21, B, N, Lkv, R, ps, [13, 6])
    o, lse = A.latent_attention(ql, qpe, bits, "bf16", 1.0, bt, L, 1, 0.3, Lkv=Lkv)
    m = 16
    reps = -(-m // N)
    qlp = np.tile(ql, (1, reps, 1))[:, :m]
    qpp = np.tile(qpe, (1, reps, 1))[:, :m]
    op, lp = A.latent_attention(qlp, qpp, bits, "bf16", 1.0, bt, L, 1, 0.3, Lkv=Lkv)
    np.testing.assert_allclose(op[:, :N], o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lp[:, :N], lse, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(op[:, N:], o[:, :m - N], rtol=1e-13, atol=1e-15)


def test_causal_flatten():
    """Row t of an Sq=4 verify block equals a single-token decode over seq_len - 3 + t keys."""
    B, N, Lkv, R, ps, Sq = 2, 3, 16, 8, 4, 4
    lens = [10, 2]
    ql, qpe, bits, bt, L = _rand_case(31, B, N, Lkv, R, ps, lens, Sq=Sq)
    o, lse = A.latent_attention(ql, qpe, bits, "bf16", 1.0, bt, L, Sq, 0.4, Lkv=Lkv)
    for b in range(B):
        for t in range(Sq):
            n = max(0, lens[b] - (Sq - 1) + t)
            tok = b * Sq + t
            o1, l1 = A.latent_attention(ql[tok:tok + 1], qpe[tok:tok + 1], bits, "bf16", 1.0,
                                        bt[b:b + 1], np.array([n]), 1, 0.4, Lkv=Lkv)
            np.testing.assert_array_equal(o1[0], o[tok])
            np.testing.assert_array_equal(l1[0], lse[tok])
    # request 1 (seq_len 2, Sq 4): rows 0 sees nothing -> o = 0, lse = -inf
    assert np.all(o[4] == 0) and np.isneginf(lse[4]).all()


def test_verify_window_golden():
    with open(os.path.join(GOLD, "verify_window.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert [A.visible_keys(c["seq_len"], c["qlen"], t) for t in range(c["qlen"])] == c["visible"]


def test_gather_rows_golden():
    with open(os.path.join(GOLD, "page_expansion.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        bt = np.array(c["block_table"])
        rows = []
        for b, L in enumerate(c["seq_lens"]):
            rows += A.gather_rows(bt, b, L, c["page_size"]).tolist()
        assert rows == c["rows"]


def test_closed_forms():
    Lkv, R, ps = 16, 8, 4
    # (i) one key: o = that key's kv_c, lse = its logit
    ql, qpe, bits, bt, L = _rand_case(51, 1, 2, Lkv, R, ps, [1])
    o, lse = A.latent_attention(ql, qpe, bits, "bf16", 1.0, bt, L, 1, 0.25, Lkv=Lkv)
    kc, kr = _keys_for(bits, bt, 0, 1, ps, Lkv)
    np.testing.assert_array_equal(o[0], np.repeat(kc, 2, 0))
    np.testing.assert_allclose(lse[0], 0.25 * (ql[0] @ kc[0] + qpe[0] @ kr[0]), rtol=1e-14)
    # (ii) zero query: uniform weights, o = mean of kv_c, lse = ln n
    ql, qpe, bits, bt, L = _rand_case(52, 1, 2, Lkv, R, ps, [7])
    o, lse = A.latent_attention(0 * ql, 0 * qpe, bits, "bf16", 1.0, bt, L, 1, 0.25, Lkv=Lkv)
    kc, _ = _keys_for(bits, bt, 0, 7, ps, Lkv)
    np.testing.assert_allclose(o[0], np.repeat(kc.mean(0)[None], 2, 0), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(7), rtol=1e-14)
    # (iii) one dominant key (logit gap >= 120): o is exactly that key's kv_c
    n = 9
    ql, qpe, bits, bt, L = _rand_case(53, 1, 1, Lkv, R, ps, [n])
    flat = bits.reshape(-1, Lkv + R)
    kc, kr = _keys_for(bits, bt, 0, n, ps, Lkv)
    jstar = 5
    row = int(bt[0, jstar // ps]) * ps + jstar % ps
    q = np.zeros((1, 1, Lkv))
    qp = np.zeros((1, 1, R))
    qp[0, 0] = 1000.0 * np.sign(kr[jstar] + 1e-30)
    o, lse = A.latent_attention(q, qp, bits, "bf16", 1.0, bt, L, 1, 1.0, Lkv=Lkv)
    s = qp[0, 0] @ kr.T
    assert np.sort(s)[-1] - np.sort(s)[-2] > 120 and int(np.argmax(s)) == jstar
    np.testing.assert_array_equal(o[0, 0], bf16_to_f64(flat[row, :Lkv]))


def test_paging_invariance():
    """Permuting physical pages and rewriting block_table leaves the result unchanged."""
    B, N, Lkv, R, ps = 3, 2, 16, 8, 4
    ql, qpe, bits, bt, L = _rand_case(61, B, N, Lkv, R, ps, [9, 4, 13])
    o, lse = A.latent_attention(ql, qpe, bits, "bf16", 1.0, bt, L, 1, 0.3, Lkv=Lkv)
    rng = np.random.default_rng(0)
    perm = rng.permutation(bits.shape[0])  # new position of old page p is perm[p]
    bits2 = np.empty_like(bits)
    bits2[perm] = bits
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    o2, lse2 = A.latent_attention(ql, qpe, bits2, "bf16", 1.0, bt2, L, 1, 0.3, Lkv=Lkv)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_kv_scale_is_applied_to_both_key_and_value():
    """fp8 path: the stored codes times kv_scale are the key and the value."""
    B, N, Lkv, R, ps = 1, 2, 16, 8, 4
    rng = np.random.default_rng(71)
    codes = rng.integers(0, 0x7E, size=(3, ps, Lkv + R)).astype(np.uint8)  # finite e4m3fn codes
    bt = np.array([[2, 0, 1]], dtype=np.int32)
    ql = rng.standard_normal((1, N, Lkv))
    qpe = rng.standard_normal((1, N, R))
    o, lse = A.latent_attention(ql, qpe, codes, "fp8", 0.125, bt, np.array([10]), 1, 0.2, Lkv=Lkv)
    from oracle.formats import e4m3fn_to_f64
    flat = e4m3fn_to_f64(codes.reshape(-1, Lkv + R))
    rows = [int(bt[0, j // ps]) * ps + j % ps for j in range(10)]
    kv = 0.125 * flat[rows]
    ref_o, ref_l = A.attention_brute(np.concatenate([ql[0], qpe[0]], 1).tolist(), kv.tolist(),
                                     kv[:, :Lkv].tolist(), 0.2)
    np.testing.assert_allclose(o[0], ref_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0], ref_l, rtol=1e-12)


def test_dsv3_dims_golden():
    with open(os.path.join(GOLD, "dsv3_dims.json")) as f:
        g = json.load(f)
    from mla_paged_decode_03_amd import inputs as gen
    assert (gen.LKV, gen.ROPE) == (g["Lkv"], g["R"])
    w = gen.workload("verify")
    assert (w.P, w.V) == (g["P"], g["V"])
    assert abs(w.scale - 1 / math.sqrt(g["P"] + g["R"])) < 1e-15
