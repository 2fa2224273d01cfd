"""Seeded synthetic inputs for MLA paged decode.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path and the CPU oracle consume what it
produces, so it must stay free of any code from either side.

Workloads (shapes follow the DeepSeek-V3 dimensions in the vLLM
``mla/common.py`` module docstring, "More Extent Definitions": Lkv=512, R=64,
P=128, V=128):

  tiny      B=1,   Sq=1, N=16,  page 16, one request of 256 keys whose 16
            pages are the first 16 entries of a seeded permutation of a
            32-page pool
  dsv3      B=64,  Sq=1, N=128, page 64, seq_lens ~ U[1024, 8192]
  longtail  B=128, Sq=1, N=16,  page 64, seq_lens log-uniform in [512, 32768]
  verify    B=32,  Sq=4, N=128, page 64, seq_lens = 4096, P=V=128, with
            q_nope / W_UK / W_UV (absorption and up-projection)
  fp8       B=256, Sq=1, N=128, page 64, seq_lens ~ U[2048, 16384], cache in
            float8 e4m3fn with one per-tensor scale max|x|/448

Recipe: metadata comes from ``numpy.random.Generator(PCG64(seed))`` in this
order: seq_lens, then one permutation of the page pool; request b takes the
next ceil(L_b/page) ids of that permutation as its block_table row, unused
entries are -1.  Values come from child generators
``default_rng([seed, tensor_id, chunk])`` as standard normals in float32,
rounded to nearest-even bf16 (tensor ids: 1 q / q_nope, 2 q_pe, 3 cache with
chunk = page id, 4 W_UK, 5 W_UV).  W_UK and W_UV are scaled by 0.02.  The
fp8 cache is quantised with scale amax/448: stored = e4m3fn(clamp(x*448/amax)).
Arrays are returned as raw bit patterns: uint16 for bf16, uint8 for fp8.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

LKV = 512
ROPE = 64
HEAD = LKV + ROPE

TID_Q, TID_QPE, TID_CACHE, TID_WUK, TID_WUV = 1, 2, 3, 4, 5


@dataclass
class Workload:
    name: str
    B: int
    Sq: int
    N: int
    page_size: int
    kv_dtype: str  # "bf16" | "fp8"
    seqlen_kind: str  # "fixed" | "uniform" | "loguniform"
    seqlen_lo: int
    seqlen_hi: int
    absorb: bool = False
    P: int = 128
    V: int = 128
    pool_pages: Optional[int] = None  # tiny: pool bigger than what is used
    seed: int = 0

    @property
    def T(self) -> int:
        return self.B * self.Sq

    @property
    def scale(self) -> float:
        # softmax scale 1/sqrt(P+R) = 1/sqrt(192) for every workload
        return 1.0 / math.sqrt(self.P + ROPE)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 16, 16, "bf16", "fixed", 256, 256, pool_pages=32, seed=1000),
    "dsv3": Workload("dsv3", 64, 1, 128, 64, "bf16", "uniform", 1024, 8192, seed=1001),
    "longtail": Workload("longtail", 128, 1, 16, 64, "bf16", "loguniform", 512, 32768, seed=1002),
    "verify": Workload("verify", 32, 4, 128, 64, "bf16", "fixed", 4096, 4096, absorb=True, seed=1003),
    "fp8": Workload("fp8", 256, 1, 128, 64, "fp8", "uniform", 2048, 16384, seed=1004),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (smaller B, another seed...)."""
    w = WORKLOADS[name]
    d = dict(w.__dict__)
    d.update(overrides)
    return Workload(**d)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest-even bfloat16 and return its 16-bit pattern."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _normals(seed: int, tid: int, chunk: int, n: int) -> np.ndarray:
    return np.random.default_rng([seed, tid, chunk]).standard_normal(n, dtype=np.float32)


def draw_seq_lens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.seqlen_kind == "fixed":
        return np.full(w.B, w.seqlen_lo, dtype=np.int32)
    if w.seqlen_kind == "uniform":
        return rng.integers(w.seqlen_lo, w.seqlen_hi, size=w.B, endpoint=True).astype(np.int32)
    if w.seqlen_kind == "loguniform":
        u = rng.uniform(math.log(w.seqlen_lo), math.log(w.seqlen_hi), size=w.B)
        return np.clip(np.floor(np.exp(u)), w.seqlen_lo, w.seqlen_hi).astype(np.int32)
    raise ValueError(w.seqlen_kind)


@dataclass
class Inputs:
    w: Workload
    seq_lens: np.ndarray  # [B] int32
    block_table: np.ndarray  # [B, max_pages] int32, -1 past the request's pages
    num_pages: int
    cache: np.ndarray  # [num_pages, ps, 576] uint16 (bf16 bits) or uint8 (e4m3fn bits)
    kv_scale: float
    q: Optional[np.ndarray] = None  # ql_nope [T, N, 512] bf16 bits (absorbed query)
    q_pe: Optional[np.ndarray] = None  # [T, N, 64] bf16 bits
    q_nope: Optional[np.ndarray] = None  # [T, N, P] bf16 bits (verify only)
    W_UK: Optional[np.ndarray] = None  # [Lkv, N, P] bf16 bits
    W_UV: Optional[np.ndarray] = None  # [Lkv, N, V] bf16 bits
    extra: dict = field(default_factory=dict)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_cache_f32(seed: int, pages: np.ndarray, ps: int) -> np.ndarray:
    """float32 normals for the listed physical pages, one child generator per page."""
    out = np.empty((len(pages), ps, HEAD), dtype=np.float32)
    per = ps * HEAD

    def work(lo_hi):
        lo, hi = lo_hi
        for i in range(lo, hi):
            out[i] = _normals(seed, TID_CACHE, int(pages[i]), per).reshape(ps, HEAD)

    n = len(pages)
    k = _threads()
    step = max(1, (n + k - 1) // k)
    with ThreadPoolExecutor(k) as ex:
        list(ex.map(work, [(i, min(n, i + step)) for i in range(0, n, step)]))
    return out


def quantize_e4m3fn(x: np.ndarray, amax: float) -> np.ndarray:
    """Per-tensor fp8 quantisation used to build the fp8 cache: bits of e4m3fn(clamp(x*448/amax))."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    inv = np.float32(448.0) / np.float32(amax)
    q = (t * float(inv)).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy()


def generate(w: Workload, seq_lens: Optional[np.ndarray] = None, poison_tail: bool = False) -> Inputs:
    """Draw every input of one decode call for workload ``w``.

    ``seq_lens`` may be given to override the drawn lengths (edge-case tests);
    the page permutation is still drawn from the same metadata generator.
    ``poison_tail`` puts NaN into slots past each request's last key (bf16 only).
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    drawn = draw_seq_lens(w, rng)
    if seq_lens is None:
        seq_lens = drawn
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (w.B,)
    ps = w.page_size
    pages_per = [(int(L) + ps - 1) // ps for L in seq_lens]
    used = int(sum(pages_per))
    num_pages = max(used, w.pool_pages or 0, 1)
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = max(1, max(pages_per))
    bt = np.full((w.B, max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per):
        bt[b, :n] = perm[off:off + n]
        off += n

    pool_f32 = _fill_cache_f32(w.seed, np.arange(num_pages), ps)
    if poison_tail:
        for b, L in enumerate(seq_lens):
            L = int(L)
            if L % ps:
                pool_f32[bt[b, L // ps], L % ps:, :] = np.nan
    kv_scale = 1.0
    if w.kv_dtype == "bf16":
        cache = f32_to_bf16_bits(pool_f32)
    elif w.kv_dtype == "fp8":
        amax = float(np.max(np.abs(pool_f32)))
        kv_scale = float(np.float32(amax) / np.float32(448.0))
        cache = quantize_e4m3fn(pool_f32, amax)
    else:
        raise ValueError(w.kv_dtype)
    del pool_f32

    T, N = w.T, w.N
    inp = Inputs(w=w, seq_lens=seq_lens, block_table=bt, num_pages=num_pages, cache=cache,
                 kv_scale=kv_scale)
    inp.q_pe = f32_to_bf16_bits(_normals(w.seed, TID_QPE, 0, T * N * ROPE).reshape(T, N, ROPE))
    if w.absorb:
        inp.q_nope = f32_to_bf16_bits(_normals(w.seed, TID_Q, 0, T * N * w.P).reshape(T, N, w.P))
        inp.W_UK = f32_to_bf16_bits(
            np.float32(0.02) * _normals(w.seed, TID_WUK, 0, LKV * N * w.P).reshape(LKV, N, w.P))
        inp.W_UV = f32_to_bf16_bits(
            np.float32(0.02) * _normals(w.seed, TID_WUV, 0, LKV * N * w.V).reshape(LKV, N, w.V))
    else:
        inp.q = f32_to_bf16_bits(_normals(w.seed, TID_Q, 0, T * N * LKV).reshape(T, N, LKV))
    return inp


def random_bf16(seed: int, tid: int, shape, scale: float = 1.0) -> np.ndarray:
    """bf16 bits of scale*N(0,1) for ad-hoc test tensors (merge inputs, GEMM operands)."""
    n = int(np.prod(shape))
    return f32_to_bf16_bits(np.float32(scale) * _normals(seed, tid, 0, n).reshape(shape))


def random_f32(seed: int, tid: int, shape, scale: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    return (np.float32(scale) * _normals(seed, tid, 0, n)).reshape(shape)


# ---- chunked prefill -------------------------------------------------------------------
TID_NEW_KV, TID_NEW_PE = 6, 7


@dataclass
class PrefillInputs:
    """One chunked-prefill batch: request b has ctx_lens[b] context tokens in the paged
    cache and new_lens[b] new tokens (rows cu_new[b] .. cu_new[b+1]-1 of the token arrays)."""
    ctx: Inputs  # cache pool, block_table, kv_scale; ctx.seq_lens = context lengths
    new_lens: np.ndarray  # [B] int32
    cu_new: np.ndarray  # [B+1] int32
    q_nope: np.ndarray  # [T, N, P] bf16 bits
    q_pe: np.ndarray  # [T, N, R] bf16 bits
    kv_c: np.ndarray  # [T, 512] bf16 bits (the new tokens' latent rows)
    k_pe: np.ndarray  # [T, 64] bf16 bits
    W_UK: np.ndarray  # [512, N, P] bf16 bits
    W_UV: np.ndarray  # [512, N, V] bf16 bits
    N: int = 128
    P: int = 128
    V: int = 128

    @property
    def T(self) -> int:
        return int(self.cu_new[-1])

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.P + ROPE)


def generate_prefill(ctx_lens, new_lens, N: int = 128, page_size: int = 64, kv_dtype: str = "bf16",
                     seed: int = 2000, P: int = 128, V: int = 128) -> PrefillInputs:
    """Seeded chunked-prefill inputs.  The context cache, block table and fp8 scale are
    drawn as for a decode batch with seq_lens = ctx_lens (same metadata generator and
    per-page value generators); the new tokens' q_nope / q_pe / kv_c / k_pe are standard
    normals (tensor ids 1, 2, 6, 7), W_UK / W_UV 0.02 * standard normals (ids 4, 5), all
    rounded to bf16."""
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    new_lens = np.asarray(new_lens, dtype=np.int32)
    B = len(ctx_lens)
    assert new_lens.shape == (B,)
    w = Workload("prefill", B, 1, N, page_size, kv_dtype, "fixed", 0, 0, P=P, V=V, seed=seed)
    ctx = generate(w, seq_lens=ctx_lens)
    ctx.q = None  # the decode query drawn by generate() is not part of a prefill batch
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(new_lens)
    T = int(cu[-1])
    nrm = lambda tid, shape, s=1.0: f32_to_bf16_bits(
        np.float32(s) * _normals(seed, tid, 0, int(np.prod(shape))).reshape(shape))
    return PrefillInputs(
        ctx=ctx, new_lens=new_lens, cu_new=cu,
        q_nope=nrm(TID_Q, (T, N, P)), q_pe=nrm(TID_QPE, (T, N, ROPE)),
        kv_c=nrm(TID_NEW_KV, (T, LKV)), k_pe=nrm(TID_NEW_PE, (T, ROPE)),
        W_UK=nrm(TID_WUK, (LKV, N, P), 0.02), W_UV=nrm(TID_WUV, (LKV, N, V), 0.02), N=N, P=P, V=V)


# The chunked-prefill workload: DeepSeek-V3 heads (N=128, P=V=128, R=64), 4 requests of
# 2048 new tokens, each after 6144 tokens of context in 64-token pages, and a context
# workspace of 8192 tokens (3 chunks of 2048 per request).
PREFILL_WORKLOAD = dict(ctx_lens=[6144] * 4, new_lens=[2048] * 4, N=128, page_size=64,
                        kv_dtype="bf16", seed=2001, workspace_tokens=8192)
