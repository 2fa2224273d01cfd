"""MLA decode in float64, written from the pages (oracle; test infrastructure only).

Notation of the ``mla/common.py`` module docstring ("More Extent
Definitions"): N heads, Lkv latent width (512), R rope width (64), P no-rope
width (128), V value width (128), Sq query tokens per request, Skv keys.

Readings where the pages leave a step open:
* The softmax scale is an explicit argument (``self.scale`` in every impl on
  the pages); the docstring's SDPA calls show none.
* LSE is natural-log and includes the scale (vLLM's merge takes
  ``is_lse_base_on_e`` true by default; flashinfer's base-2 LSE is converted).
* A query row that sees no key has o = 0 and lse = -inf; a merge of all -inf
  states is o = 0, lse = -inf.
* For Sq > 1, seq_len counts the Sq new tokens, already in the cache, and
  query row t of a request sees keys j < seq_len - (Sq - 1) + t (clamped at 0),
  as stated for multi-token verify in ``rocm_aiter_mla``,
  ``AiterMLAImpl.forward_mqa``.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

from .formats import decode


def absorb(q_nope: np.ndarray, W_UK: np.ndarray) -> np.ndarray:
    """ql_nope[t,h,l] = sum_p q_nope[t,h,p] * W_UK[l,h,p].

    ``mla/common.py`` docstring, "Data-Movement Friendly Approach": the einsum
    "snh,lnh->snl" of q_nope with W_UK [Lkv, N, P]; the layer's
    ``forward_impl`` runs it as a per-head bmm (N,B,P)x(N,P,L).
    """
    q = np.asarray(q_nope, dtype=np.float64)
    W = np.asarray(W_UK, dtype=np.float64)
    return np.einsum("tnp,lnp->tnl", q, W)


def up_proj(o_latent: np.ndarray, W_UV: np.ndarray) -> np.ndarray:
    """o[t,h,v] = sum_l o_latent[t,h,l] * W_UV[l,h,v].

    ``mla/common.py`` docstring, "Data-Movement Friendly Approach": the einsum
    "snl,lnv->snv"; the layer's ``_v_up_proj`` runs it as bmm (N,B,L)x(N,L,V).
    """
    o = np.asarray(o_latent, dtype=np.float64)
    W = np.asarray(W_UV, dtype=np.float64)
    return np.einsum("tnl,lnv->tnv", o, W)


def gather_rows(block_table: np.ndarray, b: int, n: int, page_size: int) -> np.ndarray:
    """Physical cache rows of keys 0..n-1 of request b.

    A block_table entry e covering ``page_size`` tokens expands to the flat rows
    e*page_size ... e*page_size + page_size - 1 (``rocm_aiter_mla``,
    ``AiterMLAMetadataBuilder._build_decode``, page-index expansion).
    """
    rows = np.empty(n, dtype=np.int64)
    for j in range(n):
        rows[j] = int(block_table[b, j // page_size]) * page_size + j % page_size
    return rows


def visible_keys(seq_len: int, Sq: int, t: int) -> int:
    """Keys seen by query row t of a request (causal multi-token verify window)."""
    return max(0, int(seq_len) - (Sq - 1) + t)


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Softmax attention of rows q [M, D] over keys [n, D] / values [n, Dv].

    Returns (o [M, Dv], lse [M]).  For n = 0: o = 0, lse = -inf.
    """
    M = q.shape[0]
    n = keys.shape[0]
    if n == 0:
        return np.zeros((M, values.shape[1])), np.full(M, -np.inf)
    s = scale * (q @ keys.T)  # [M, n]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(axis=1, keepdims=True)
    o = (p @ values) / z
    lse = (m + np.log(z))[:, 0]
    return o, lse


def latent_attention(ql_nope: np.ndarray, q_pe: np.ndarray, cache_bits: np.ndarray,
                     cache_dtype: str, kv_scale: float, block_table: np.ndarray,
                     seq_lens: np.ndarray, Sq: int, scale: float,
                     requests: Optional[Iterable[int]] = None, Lkv: int = 512):
    """Absorbed MLA decode: MQA with QK dim Lkv+R over one shared latent head.

    ``mla/common.py`` docstring, "Data-Movement Friendly Approach":
    spda_o = SDPA(cat[ql_nope, q_pe], cat[kv_c, k_pe], kv_c), i.e. every head
    attends over the same cache rows [kv_c | k_pe], and the value is kv_c
    (V head dim = Lkv).  A cache row holds kv_c in its first Lkv entries and
    k_pe after it (``rocm_aiter_mla``, ``forward_mqa``: kv_pe_offset =
    kv_lora_rank).  Stored fp8 values are multiplied by ``kv_scale``.

    ql_nope [T, N, Lkv], q_pe [T, N, R] float64 (token t = b*Sq + i);
    cache_bits [pages, page_size, Lkv+R] raw bits.  Returns o [T, N, Lkv] and
    lse [T, N]; rows of requests not listed in ``requests`` are NaN.
    """
    T, N, _ = ql_nope.shape
    ps = cache_bits.shape[1]
    B = len(seq_lens)
    assert T == B * Sq
    o = np.full((T, N, Lkv), np.nan)
    lse = np.full((T, N), np.nan)
    reqs = range(B) if requests is None else requests
    for b in reqs:
        L = int(seq_lens[b])
        rows = gather_rows(block_table, b, L, ps)
        flat = cache_bits.reshape(-1, cache_bits.shape[2])
        kv = decode(flat[rows], cache_dtype) * kv_scale if L else np.zeros((0, cache_bits.shape[2]))
        kv_c, k_pe = kv[:, :Lkv], kv[:, Lkv:]
        for i in range(Sq):
            t = b * Sq + i
            n = visible_keys(L, Sq, i)
            q = np.concatenate([ql_nope[t], q_pe[t]], axis=1)  # [N, Lkv+R]
            k = np.concatenate([kv_c[:n], k_pe[:n]], axis=1)
            o[t], lse[t] = attend(q, k, kv_c[:n], scale)
    return o, lse


def merge_states(outs, lses):
    """Combine partial attention states over disjoint key sets.

    m = max_i lse_i, w_i = exp(lse_i - m), o = sum w_i o_i / sum w_i,
    lse = m + ln sum w_i; where every lse_i is -inf: o = 0, lse = -inf.
    This is the ``merge_attn_states(prefix, suffix)`` combiner of the
    ``mla/common.py`` docstring, "Chunked Prefill", applied to any number of
    parts.  outs[i] [..., D], lses[i] [...].
    """
    lse_st = np.stack([np.asarray(x, dtype=np.float64) for x in lses])  # [k, ...]
    o_st = np.stack([np.asarray(x, dtype=np.float64) for x in outs])  # [k, ..., D]
    m = lse_st.max(axis=0)
    dead = np.isneginf(m)
    m_safe = np.where(dead, 0.0, m)
    w = np.exp(lse_st - m_safe)  # exp(-inf) = 0 for empty parts
    w = np.where(dead[None], 0.0, w)
    z = w.sum(axis=0)
    z_safe = np.where(dead, 1.0, z)
    o = (w[..., None] * o_st).sum(axis=0) / z_safe[..., None]
    o = np.where(dead[..., None], 0.0, o)
    lse = np.where(dead, -np.inf, m_safe + np.log(z_safe))
    return o, lse


def mha_compute_friendly(q_nope: np.ndarray, q_pe: np.ndarray, kv_c: np.ndarray,
                         k_pe: np.ndarray, W_UK: np.ndarray, W_UV: np.ndarray,
                         scale: float, Sq: int):
    """The compute-friendly (MHA) path for one request, for cross-checking.

    Follows the ``mla/common.py`` module docstring, section "Compute Friendly
    Approach": every cache row's latent vector is up-projected per head, giving
    the key part k_nope[j,h,:] = sum_l kv_c[j,l] W_UK[l,h,:] and the value
    v[j,h,:] = sum_l kv_c[j,l] W_UV[l,h,:]; each head then runs plain softmax
    attention with query [q_nope | q_pe] (width P+R) against keys [k_nope | k_pe],
    the rope part of the key being the same for all heads.
    q_nope [Sq, N, P], q_pe [Sq, N, R], kv_c [L, Lkv], k_pe [L, R].
    Returns o [Sq, N, V], lse [Sq, N].
    """
    Lkv, N, P = W_UK.shape
    V = W_UV.shape[2]
    L = kv_c.shape[0]
    k_nope = (kv_c @ W_UK.reshape(Lkv, N * P)).reshape(L, N, P)
    v = (kv_c @ W_UV.reshape(Lkv, N * V)).reshape(L, N, V)
    o = np.zeros((Sq, N, V))
    lse = np.zeros((Sq, N))
    for i in range(Sq):
        n = visible_keys(L, Sq, i)
        for h in range(N):
            q = np.concatenate([q_nope[i, h], q_pe[i, h]])[None]
            k = np.concatenate([k_nope[:n, h], k_pe[:n]], axis=1)
            oo, ll = attend(q, k, v[:n, h], scale)
            o[i, h], lse[i, h] = oo[0], ll[0]
    return o, lse


def attention_brute(q_rows, keys, values, scale):
    """Scalar-loop softmax attention without max subtraction (tiny inputs only)."""
    out = []
    lses = []
    for q in q_rows:
        ws = []
        for k in keys:
            d = 0.0
            for a, c in zip(q, k):
                d += a * c
            ws.append(math.exp(scale * d))
        z = sum(ws)
        o = [0.0] * len(values[0])
        for w_, vrow in zip(ws, values):
            for c in range(len(o)):
                o[c] += w_ * vrow[c]
        out.append([x / z for x in o])
        lses.append(math.log(z))
    return np.array(out), np.array(lses)
