"""Chunked prefill over a paged latent cache, compute-friendly form (oracle; test
infrastructure only).

Sources: vLLM ``v1/attention/backends/mla/common.py``:

* the module docstring, section "Chunked Prefill": the new tokens attend to their own
  keys causally, then to the existing context in chunks of at most MCC tokens, and the
  partial outputs are combined with ``merge_attn_states``; keys and values of every
  token are up-projected from its latent row, k_nope = kv_c @ W_UK and
  v = kv_c @ W_UV, and k_pe is shared by all heads;
* ``MLACommonImpl._compute_prefill_context``: one chunk = gather (and dequantise with
  the cache scale) the chunk's latent rows of every request into a workspace, then
  ``kv_b_proj``, then a non-causal attention of all new tokens against the chunk;
* ``MLACommonImpl.forward_mha``: the new tokens' causal attention, then one merge of the
  context output (prefix) with it (suffix);
* ``MLACommonMetadataBuilder``, chunked-context metadata: the workspace is split evenly
  over the requests that have context (rounded down to a multiple of the page size), and
  chunk i of request b covers context positions [i*MCC, min((i+1)*MCC, C_b)).

What the path computes is plain attention, so ``chunked_prefill`` is that definition:
request b has C_b context tokens (in the paged cache) followed by S_b new tokens; new
token i sits at position C_b + i and sees every key at a position <= C_b + i.  The
chunk loop is a way to compute it in bounded memory; ``tests/test_oracle_prefill.py``
checks the loop (written from the docstring, with ``attention.merge_states``) against
this definition.

Readings where the pages leave a step open:
* The context comes from the cache dequantised (value * kv_scale for fp8), the new
  tokens' latent rows are used as given (bf16): ``forward_mha`` up-projects
  ``kv_c_normed`` of the new tokens directly, not a copy read back from the cache.
* LSE is natural-log and includes the scale, laid out [T, N] (token-major), the layout
  the decode path uses; the docstring's [N, Sq] is a property of the library it calls.
* A row with no visible key has o = 0 and lse = -inf (only possible with S_b = 0 rows,
  i.e. never for a real query, and for a context chunk a request has no tokens in).
"""
from __future__ import annotations

import numpy as np

from .attention import attend, gather_rows
from .formats import decode, round_to_bf16


def chunk_plan(ctx_lens, workspace_tokens: int, page_size: int):
    """Chunk schedule of the context (``MLACommonMetadataBuilder`` chunked context).

    MCC = workspace_tokens // (number of requests with context), rounded down to a
    multiple of page_size (kept as is when that would give 0); n_chunks =
    ceil(max C_b / MCC).  Returns (mcc, starts [n, B], lens [n, B], cu [n, B+1]).
    No context at all: mcc = 0 and no chunks.
    """
    C = np.asarray(ctx_lens, dtype=np.int64)
    B = len(C)
    with_ctx = int((C > 0).sum())
    if with_ctx == 0:
        return 0, np.zeros((0, B), np.int64), np.zeros((0, B), np.int64), np.zeros((0, B + 1), np.int64)
    mcc = workspace_tokens // with_ctx
    if mcc >= page_size:
        mcc = (mcc // page_size) * page_size
    if mcc <= 0:
        raise ValueError("workspace smaller than the number of requests with context")
    n = -(-int(C.max()) // mcc)
    starts = np.arange(n, dtype=np.int64)[:, None] * mcc * np.ones((1, B), np.int64)
    ends = np.minimum(C[None, :], starts + mcc)
    lens = np.maximum(ends - starts, 0)
    cu = np.zeros((n, B + 1), np.int64)
    cu[:, 1:] = np.cumsum(lens, axis=1)
    return mcc, starts, lens, cu


def context_rows(cache_bits, cache_dtype: str, kv_scale: float, block_table, b: int,
                 start: int, n: int) -> np.ndarray:
    """Latent rows [n, 576] (float64) of context positions start..start+n-1 of request b,
    read through the block table and dequantised (``gather_and_maybe_dequant_cache``)."""
    ps = cache_bits.shape[1]
    rows = gather_rows(block_table, b, start + n, ps)[start:]
    flat = cache_bits.reshape(-1, cache_bits.shape[2])
    if n == 0:
        return np.zeros((0, cache_bits.shape[2]))
    return decode(flat[rows], cache_dtype) * (kv_scale if cache_dtype != "bf16" else 1.0)


def kv_b_proj(kv_c: np.ndarray, W_UK: np.ndarray, W_UV: np.ndarray, round_to=None):
    """k_nope[s,h,p] = sum_l kv_c[s,l] W_UK[l,h,p];  v[s,h,c] = sum_l kv_c[s,l] W_UV[l,h,c]
    (docstring "Chunked Prefill": new_k_nope / new_v, cache_k_nope_chunk / cache_v_chunk).

    round_to="bf16" rounds both results to bfloat16 (ties to even): the pages materialise
    k_nope and v as the output of the kv_b_proj linear layer, in the model's dtype
    (``_compute_prefill_context`` and ``forward_mha`` split ``kv_b_proj(...)``), so every
    logit of that pipeline is taken against the rounded keys."""
    Lkv, N, P = W_UK.shape
    V = W_UV.shape[2]
    S = kv_c.shape[0]
    k_nope = (kv_c @ W_UK.reshape(Lkv, N * P)).reshape(S, N, P)
    v = (kv_c @ W_UV.reshape(Lkv, N * V)).reshape(S, N, V)
    if round_to == "bf16":
        k_nope, v = round_to_bf16(k_nope), round_to_bf16(v)
    elif round_to is not None:
        raise ValueError(round_to)
    return k_nope, v


def mha(q_nope, q_pe, k_nope, k_pe, v, scale: float, causal: bool):
    """Per-head attention of one request: q [Sq, N, P|R], k_nope [Sk, N, P], k_pe [Sk, R]
    (all heads), v [Sk, N, V].  Causal: query i sees keys j <= i + Sk - Sq (the new tokens
    are the last Sq of the Sk keys).  Returns o [Sq, N, V], lse [Sq, N]."""
    Sq, N, _ = q_nope.shape
    Sk = k_nope.shape[0]
    V = v.shape[2]
    o = np.zeros((Sq, N, V))
    lse = np.zeros((Sq, N))
    for h in range(N):
        q = np.concatenate([q_nope[:, h], q_pe[:, h]], axis=1)  # [Sq, P+R]
        k = np.concatenate([k_nope[:, h], k_pe], axis=1)  # [Sk, P+R]
        if not causal:
            o[:, h], lse[:, h] = attend(q, k, v[:, h], scale)
            continue
        for i in range(Sq):
            n = max(0, min(Sk, i + Sk - Sq + 1))
            oo, ll = attend(q[i:i + 1], k[:n], v[:n, h], scale)
            o[i, h], lse[i, h] = oo[0], ll[0]
    return o, lse


def chunked_prefill(q_nope, q_pe, cu_new, kv_c, k_pe, ctx_lens, cache_bits, cache_dtype: str,
                    kv_scale: float, block_table, W_UK, W_UV, scale: float, requests=None,
                    kv_round=None):
    """Output of a chunked-prefill batch, by the definition.

    q_nope [T, N, P], q_pe [T, N, R], kv_c [T, Lkv], k_pe [T, R] (float64, the T new tokens,
    request b owning rows cu_new[b]..cu_new[b+1]-1); ctx_lens [B] context lengths, whose
    latent rows are in the paged cache ``cache_bits`` [pages, ps, Lkv+R] through
    ``block_table``.  Returns o [T, N, V], lse [T, N]; rows of requests not listed in
    ``requests`` are NaN.

    kv_round="bf16" keeps the pipeline's intermediate tensors in the model dtype, as the
    pages hold them: the dequantised context rows (the bf16 workspace that
    ``gather_and_maybe_dequant_cache`` fills) and k_nope, v (the output of ``kv_b_proj``),
    each rounded to bfloat16, ties to even.  None computes the definition unrounded.
    """
    Lkv = W_UK.shape[0]
    T, N, _ = q_nope.shape
    V = W_UV.shape[2]
    o = np.full((T, N, V), np.nan)
    lse = np.full((T, N), np.nan)
    B = len(ctx_lens)
    for b in (range(B) if requests is None else requests):
        lo, hi = int(cu_new[b]), int(cu_new[b + 1])
        C = int(ctx_lens[b])
        ctx = context_rows(cache_bits, cache_dtype, kv_scale, block_table, b, 0, C)
        if kv_round == "bf16":
            ctx = round_to_bf16(ctx)
        lat = np.concatenate([ctx[:, :Lkv], kv_c[lo:hi]], axis=0)
        pe = np.concatenate([ctx[:, Lkv:], k_pe[lo:hi]], axis=0)
        k_nope, v = kv_b_proj(lat, W_UK, W_UV, round_to=kv_round)
        o[lo:hi], lse[lo:hi] = mha(q_nope[lo:hi], q_pe[lo:hi], k_nope, pe, v, scale, causal=True)
    return o, lse
