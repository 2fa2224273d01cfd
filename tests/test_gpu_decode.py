"""GPU parity of the HIP decode path against the fp64 oracle, through the C ABI.

Small cases compare every output element; they span several 32-key tiles, ragged
tails, empty requests, page sizes that do and do not divide the tile, head
counts 1..128, 1..8 query tokens, bf16 and fp8 caches, split and unsplit plans.
Tolerances: bf16 output max-abs <= 1e-2 and rel-L2 <= 5e-3; LSE max-abs <= 1e-3.
Integer work (plan, gather rows) is compared bit-exactly.
"""
import math

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


def _api():
    from mla_paged_decode_03_amd import api
    return api


def run_decode(torch, inp, num_cus=0, with_lse=True, poison_bt=False):
    """Uploads one decode problem, plans, runs; returns (o [T,N,512] f64, lse [T,N] f64, plan)."""
    api = _api()
    w = inp.w
    dev = "cuda"
    q = bf16_dev(inp.q)
    q_pe = bf16_dev(inp.q_pe)
    cache = bf16_dev(inp.cache) if w.kv_dtype == "bf16" else u8_dev(inp.cache)
    bt_np = inp.block_table.copy()
    if poison_bt:
        bt_np[bt_np < 0] = -1
    bt = torch.from_numpy(bt_np).to(dev)
    sl = torch.from_numpy(inp.seq_lens).to(dev)
    T, N = w.T, w.N
    o = torch.full((T, N, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((T, N), float("nan"), dtype=torch.float32, device=dev) if with_lse else None
    dt = api.MLA_DT_BF16 if w.kv_dtype == "bf16" else api.MLA_DT_FP8_E4M3FN
    plan = api.mla_decode_plan(inp.seq_lens, w.Sq, N, w.page_size, bt_np.shape[1], dt, num_cus)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    api.mla_decode_run(plan, q, q_pe, cache, bt, sl, w.scale, inp.kv_scale, o, lse, ws)
    torch.cuda.synchronize()
    return bf16_host(o), (lse.cpu().numpy().astype(np.float64) if with_lse else None), plan


def oracle(inp, requests=None):
    from oracle import attention as A
    from oracle.formats import bf16_to_f64
    w = inp.w
    return A.latent_attention(bf16_to_f64(inp.q), bf16_to_f64(inp.q_pe), inp.cache, w.kv_dtype,
                              inp.kv_scale, inp.block_table, inp.seq_lens, w.Sq, w.scale,
                              requests=requests)


def elem_bound(ref):
    """Per-element bound on |o - ref|: max-abs 1e-2, plus half a bf16 ulp of ref where
    |ref| >= 4.  There the final rounding of o to bf16 alone can move an element by
    half an ulp (2^-6 for |ref| in [4, 8)), more than 1e-2; below 4 that rounding is at
    most 2^-7 and the plain 1e-2 bound holds."""
    a = np.abs(ref)
    half_ulp = np.ldexp(1.0, np.frexp(np.where(a > 0, a, 1.0))[1] - 9)  # bf16: 8 significant bits
    return O_MAX_ABS + np.where(a >= 4.0, half_ulp, 0.0)


def check(o, lse, ro, rl, rows=None):
    """Parity against the oracle: every element within elem_bound (max-abs 1e-2, plus half
    a bf16 ulp of the reference where |ref| >= 4), rel-L2 <= 5e-3, LSE within 1e-3 and
    the same -inf pattern.  Prints the achieved errors."""
    if rows is not None:
        o, lse, ro, rl = o[rows], lse[rows], ro[rows], rl[rows]
    assert np.all(np.isfinite(o))
    ma, rel = metrics(o, ro)
    fin = np.isfinite(rl)
    lerr = float(np.max(np.abs(lse[fin] - rl[fin]))) if (lse is not None and fin.any()) else 0.0
    over = np.abs(o - ro) > elem_bound(ro)
    big = np.abs(ro) >= 4.0
    ma_small = float(np.max(np.abs(o - ro)[~big])) if (~big).any() else 0.0
    info = dict(max_abs=ma, max_abs_below_4=ma_small, rel_l2=rel, lse_max_abs=lerr, elems_ref_ge_4=int(big.sum()))
    print("parity", info, flush=True)
    assert not over.any() and rel <= O_REL_L2, info
    if lse is not None:
        assert np.array_equal(fin, np.isfinite(lse)), "LSE -inf pattern differs"
        assert np.all(lse[~fin] == -np.inf)
        assert lerr <= LSE_MAX_ABS, info
    return info


def gen_case(name="tiny", seq_lens=None, **kw):
    from mla_paged_decode_03_amd import inputs as gen
    w = gen.workload(name, **kw)
    return gen.generate(w, seq_lens=seq_lens)


def test_tiny_workload_full_parity(torch_cuda):
    inp = gen_case("tiny")
    o, lse, _ = run_decode(torch_cuda, inp)
    ro, rl = oracle(inp)
    check(o, lse, ro, rl)


CASES = [
    # (N, Sq, page_size, seq_lens, kv dtype, num_cus)
    (16, 1, 16, [256], "bf16", 0),
    (16, 1, 64, [1, 31, 32, 33, 64, 65, 300], "bf16", 0),
    (128, 1, 64, [70, 1000, 5], "bf16", 0),
    (128, 1, 64, [2000, 700, 64], "bf16", 4),      # forced splits
    (48, 1, 16, [0, 77, 129], "bf16", 2),           # empty request, NRB=2
    (100, 1, 32, [513, 64], "bf16", 3),             # NRB=4 with padded rows
    (128, 4, 64, [300, 4, 3, 1], "bf16", 0),        # causal verify, rows seeing nothing
    (16, 4, 16, [90, 7], "bf16", 5),                # Sq*N = 64 rows, split
    (32, 8, 64, [200, 10], "bf16", 0),              # Sq=8 -> 256 rows, 2 head groups
    (1, 1, 1, [1, 2, 40], "bf16", 0),               # one head, page size 1
    (8, 2, 7, [50, 13], "bf16", 2),                 # odd page size
    (128, 1, 64, [300, 1000], "fp8", 0),
    (16, 1, 64, [4000, 100], "fp8", 6),
    (128, 4, 64, [257, 2], "fp8", 3),
    (128, 1, 16, [300, 1000], "fp8", 0),            # fp8, generic pages (16 keys)
    (16, 2, 7, [90, 13], "fp8", 3),                 # fp8, odd page size, split
    (32, 1, 1, [5, 70], "fp8", 2),                  # fp8, page size 1
]


@pytest.mark.parametrize("N,Sq,ps,lens,dt,cus", CASES)
def test_parity_small(torch_cuda, N, Sq, ps, lens, dt, cus):
    name = "fp8" if dt == "fp8" else "tiny"
    inp = gen_case(name, seq_lens=np.array(lens, np.int32), B=len(lens), N=N, Sq=Sq, page_size=ps,
                   pool_pages=None, seed=77 + N + Sq + ps)
    o, lse, plan = run_decode(torch_cuda, inp, num_cus=cus)
    ro, rl = oracle(inp)
    check(o, lse, ro, rl)


def test_plan_export_bit_exact(torch_cuda):
    from oracle import plan as PL
    api = _api()
    rng = np.random.default_rng(5)
    for Sq, N, cus in [(1, 128, 256), (4, 128, 256), (1, 16, 256), (2, 40, 17)]:
        L = rng.integers(0, 20000, size=97).astype(np.int32)
        plan = api.mla_decode_plan(L, Sq, N, 64, 400, api.MLA_DT_BF16, cus)
        w, r = api.mla_plan_export(plan)
        p = PL.split_plan(L, Sq, N, cus)
        assert np.array_equal(w, np.array(p["items"], np.int32).reshape(-1, 5))
        assert np.array_equal(r, np.array(p["reduce"], np.int32).reshape(-1, 3))
        assert plan.workspace_bytes == PL.workspace_bytes(p["num_partials"], Sq, N)
        plan.destroy()


def test_gather_rows_bit_exact(torch_cuda):
    from oracle import plan as PL
    torch = torch_cuda
    api = _api()
    for ps, lens in [(64, [1, 64, 65, 3000]), (16, [256]), (1, [5, 0, 9]), (7, [50, 13])]:
        inp = gen_case("tiny", seq_lens=np.array(lens, np.int32), B=len(lens), page_size=ps,
                       pool_pages=None)
        plan = api.mla_decode_plan(inp.seq_lens, 1, 16, ps, inp.block_table.shape[1])
        total = int(inp.seq_lens.sum())
        rows = torch.full((max(total, 1),), -7, dtype=torch.int64, device="cuda")
        api.mla_debug_gather_rows(plan, torch.from_numpy(inp.block_table).cuda(), rows)
        torch.cuda.synchronize()
        exp = PL.gather_rows_all(inp.block_table, inp.seq_lens, ps)
        assert rows.cpu().numpy()[:total].tolist() == exp


def test_paging_invariance_bitwise(torch_cuda):
    inp = gen_case("tiny", seq_lens=np.array([700, 129, 64], np.int32), B=3, N=128, page_size=64,
                   pool_pages=None, seed=11)
    ro, rl = oracle(inp)
    o1, l1, _ = run_decode(torch_cuda, inp)
    perm = np.random.default_rng(3).permutation(inp.num_pages)
    cache2 = np.empty_like(inp.cache)
    cache2[perm] = inp.cache
    inp.cache = cache2
    inp.block_table = np.where(inp.block_table >= 0, perm[np.maximum(inp.block_table, 0)],
                               -1).astype(np.int32)
    o2, l2, _ = run_decode(torch_cuda, inp)
    o3, l3, _ = run_decode(torch_cuda, inp, num_cus=1)
    for name, (o, l) in dict(orig=(o1, l1), perm=(o2, l2), perm_unsplit=(o3, l3)).items():
        per_req = [metrics(o[b], ro[b]) for b in range(3)]
        print(name, per_req, flush=True)
    check(o1, l1, ro, rl)
    check(o2, l2, ro, rl)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_head_independence_bitwise(torch_cuda):
    """Extra query heads leave the real heads bit-identical (same row-block shape, same plan)."""
    lens = np.array([900, 40], np.int32)
    inp = gen_case("tiny", seq_lens=lens, B=2, N=128, page_size=64, pool_pages=None, seed=13)
    o_full, l_full, _ = run_decode(torch_cuda, inp)
    small = gen_case("tiny", seq_lens=lens, B=2, N=100, page_size=64, pool_pages=None, seed=13)
    small.cache, small.block_table = inp.cache, inp.block_table
    small.q = np.ascontiguousarray(inp.q[:, :100])
    small.q_pe = np.ascontiguousarray(inp.q_pe[:, :100])
    o_s, l_s, _ = run_decode(torch_cuda, small)
    assert np.array_equal(o_s, o_full[:, :100]) and np.array_equal(l_s, l_full[:, :100])


def test_split_matches_unsplit(torch_cuda):
    inp = gen_case("tiny", seq_lens=np.array([5000, 3000], np.int32), B=2, N=128, page_size=64,
                   pool_pages=None, seed=17)
    o1, l1, p1 = run_decode(torch_cuda, inp, num_cus=1)
    o2, l2, p2 = run_decode(torch_cuda, inp, num_cus=64)
    assert p1.workspace_bytes == 0 and p2.workspace_bytes > 0
    # one bf16 rounding apart at most: the split path rounds the merged fp32 states once
    assert np.all(np.abs(o1 - o2) <= 2.0 ** -7 * np.maximum(np.abs(o1), np.abs(o2)) + 1e-3)
    assert metrics(o1, o2)[1] <= 3e-3
    assert np.max(np.abs(l1 - l2)) <= 1e-4


def test_poisoned_tail_and_table(torch_cuda):
    """NaN in slots past seq_len and -1 in unused block_table entries never reach the output."""
    from mla_paged_decode_03_amd import inputs as gen
    w = gen.workload("tiny", B=3, N=16, page_size=64, pool_pages=None, seed=19)
    inp = gen.generate(w, seq_lens=np.array([100, 63, 1], np.int32), poison_tail=True)
    o, lse, _ = run_decode(torch_cuda, inp, poison_bt=True)
    clean = gen.generate(w, seq_lens=np.array([100, 63, 1], np.int32))
    ro, rl = oracle(clean)
    check(o, lse, ro, rl)


def test_dominant_key_exact(torch_cuda):
    """A key whose logit leads by >= 120 gets all the weight: o equals its kv_c bitwise."""
    from oracle.formats import bf16_to_f64
    inp = gen_case("tiny", seq_lens=np.array([333], np.int32), B=1, N=16, page_size=64,
                   pool_pages=None, seed=23)
    j = 201
    row = int(inp.block_table[0, j // 64]) * 64 + j % 64
    flat = inp.cache.reshape(-1, 576)
    kpe = bf16_to_f64(flat[row, 512:])
    inp.q = np.zeros_like(inp.q)
    # q_pe aligned with the key's rope part, large enough to dominate every other key
    scale_up = 8000.0 / max(1e-6, np.abs(kpe).sum())
    from mla_paged_decode_03_amd.inputs import f32_to_bf16_bits
    qpe = (np.sign(kpe) * scale_up).astype(np.float32)
    inp.q_pe = np.broadcast_to(f32_to_bf16_bits(qpe), inp.q_pe.shape).copy()
    o, lse, _ = run_decode(torch_cuda, inp)
    exp = bf16_to_f64(flat[row, :512])
    assert np.array_equal(o[0], np.broadcast_to(exp, o[0].shape))


def test_no_lse_pointer(torch_cuda):
    inp = gen_case("tiny")
    o, _, _ = run_decode(torch_cuda, inp, with_lse=False)
    ro, rl = oracle(inp)
    ma, rel = metrics(o, ro)
    assert ma <= O_MAX_ABS and rel <= O_REL_L2


def test_deterministic(torch_cuda):
    inp = gen_case("tiny", seq_lens=np.array([3000, 100], np.int32), B=2, N=128, page_size=64,
                   pool_pages=None, seed=29)
    a = run_decode(torch_cuda, inp, num_cus=16)
    b = run_decode(torch_cuda, inp, num_cus=16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_workspace_too_small_is_rejected(torch_cuda):
    torch = torch_cuda
    api = _api()
    inp = gen_case("tiny", seq_lens=np.array([3000], np.int32), B=1, N=16, page_size=64,
                   pool_pages=None)
    plan = api.mla_decode_plan(inp.seq_lens, 1, 16, 64, inp.block_table.shape[1], num_cus=8)
    assert plan.workspace_bytes > 0
    q, qpe, cache = bf16_dev(inp.q), bf16_dev(inp.q_pe), bf16_dev(inp.cache)
    bt = torch.from_numpy(inp.block_table).cuda()
    sl = torch.from_numpy(inp.seq_lens).cuda()
    o = torch.empty((1, 16, 512), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(plan.workspace_bytes - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(api.MLAError) as e:
        api.mla_decode_run(plan, q, qpe, cache, bt, sl, 0.1, 1.0, o, None, ws)
    assert e.value.status == api.MLA_ERR_WORKSPACE


def test_causal_flatten_on_gpu(torch_cuda):
    """Multi-token verify: query row t of an Sq = 4 decode equals an Sq = 1 decode of the
    same query over seq_len - 3 + t keys (the causal window of the rocm_aiter_mla page's
    multi-token decode).  Both unsplit (num_cus = 1), so the keys go through the same tiles
    in the same order: at most one bf16 rounding apart, LSE to fp32 rounding."""
    import copy
    import dataclasses
    lens = np.array([300, 97, 64], np.int32)
    inp = gen_case("tiny", seq_lens=lens, B=3, Sq=4, N=16, page_size=16, pool_pages=None, seed=29)
    o4, l4, _ = run_decode(torch_cuda, inp, num_cus=1)
    for t in range(4):
        one = copy.deepcopy(inp)
        one.w = dataclasses.replace(inp.w, Sq=1)
        one.seq_lens = (lens - 3 + t).astype(np.int32)
        one.q = np.ascontiguousarray(inp.q.reshape(3, 4, 16, 512)[:, t])
        one.q_pe = np.ascontiguousarray(inp.q_pe.reshape(3, 4, 16, 64)[:, t])
        o1, l1, _ = run_decode(torch_cuda, one, num_cus=1)
        a = o4.reshape(3, 4, 16, 512)[:, t]
        assert np.all(np.abs(a - o1) <= 2.0 ** -8 * np.maximum(np.abs(a), np.abs(o1)) + 1e-6), t
        assert np.max(np.abs(l4.reshape(3, 4, 16)[:, t] - l1)) <= 1e-5, t


def test_canaries_around_workspace_and_output(torch_cuda):
    """Canary words around the workspace and around o_latent / lse (plus the gaps of a padded
    head stride) are left untouched by a split run, attend and reduce included."""
    torch = torch_cuda
    api = _api()
    inp = gen_case("tiny", seq_lens=np.array([3000, 77, 1500], np.int32), B=3, N=40, page_size=64,
                   pool_pages=None, seed=31)
    w = inp.w
    T, N = w.T, w.N
    plan = api.mla_decode_plan(inp.seq_lens, w.Sq, N, w.page_size, inp.block_table.shape[1], num_cus=12)
    assert plan.workspace_bytes > 0
    PAD = 4096
    canary = 0xA5
    ws_all = torch.full((plan.workspace_bytes + 2 * PAD,), canary, dtype=torch.uint8, device="cuda")
    ws = ws_all[PAD:PAD + plan.workspace_bytes]
    hs = 520  # head stride: 8 unused elements after each 512-wide row
    o_all = torch.full((T * N * hs + 2 * PAD,), -7.0, dtype=torch.bfloat16, device="cuda")
    o = o_all[PAD:PAD + T * N * hs].view(T, N, hs)[:, :, :512]
    lse_all = torch.full((T * N + 2 * PAD,), -7.0, dtype=torch.float32, device="cuda")
    lse = lse_all[PAD:PAD + T * N].view(T, N)
    api.mla_decode_run(plan, bf16_dev(inp.q), bf16_dev(inp.q_pe), bf16_dev(inp.cache),
                       torch.from_numpy(inp.block_table).cuda(), torch.from_numpy(inp.seq_lens).cuda(),
                       w.scale, inp.kv_scale, o, lse, ws)
    torch.cuda.synchronize()
    wsh = ws_all.cpu().numpy()
    assert np.all(wsh[:PAD] == canary) and np.all(wsh[-PAD:] == canary)
    oh = o_all.float().cpu().numpy()
    assert np.all(oh[:PAD] == -7.0) and np.all(oh[-PAD:] == -7.0)
    gaps = oh[PAD:PAD + T * N * hs].reshape(T, N, hs)[:, :, 512:]
    assert np.all(gaps == -7.0)
    lh = lse_all.cpu().numpy()
    assert np.all(lh[:PAD] == -7.0) and np.all(lh[-PAD:] == -7.0)
    ro, rl = oracle(inp)
    check(bf16_host(o), lse.cpu().numpy().astype(np.float64), ro, rl)
    plan.destroy()


@pytest.mark.parametrize("ps,L,cus", [
    (64, 1000, 3),    # tile-aligned pages (one base per tile), segments cut at 64-key granules
    (32, 333, 2),     # one page per tile
    (128, 700, 5),    # two tiles per page
    (64, 97, 0),      # one unsplit request ending inside its second tile
    (16, 600, 3),     # pages smaller than a tile: per-row block-table lookups
])
def test_gather_addressing_dominant_keys(torch_cuda, ps, L, cus):
    """The decode kernel's own addressing, without the test-only gather kernel: query head h
    is aligned with the rope part of key j_h only, so key j_h carries all the weight (the
    other logits trail by hundreds of log2 units and their exponentials underflow to 0)
    and o[h] must equal that key's latent row bit for bit.  The 16 keys sit at tile,
    page, granule and segment boundaries and in the last partial tile, so a wrong tile
    base, lane offset or end-of-segment clamp shows as a different row.  Split plans
    (cus > 0) also run the fp16 partials and the reduce, which keep a single key exact."""
    from oracle.formats import bf16_to_f64
    from mla_paged_decode_03_amd.inputs import f32_to_bf16_bits
    inp = gen_case("tiny", seq_lens=np.array([L], np.int32), B=1, N=16, page_size=ps, pool_pages=None,
                   seed=600 + ps + L)
    cands = [0, 1, 31, 32, 33, 63, 64, 65, L - 1, L - 2, (L - 1) // 32 * 32, L // 2, 127, 128, 191, 192]
    js = [min(max(j, 0), L - 1) for j in cands][:16]
    flat = inp.cache.reshape(-1, 576)
    rows = [int(inp.block_table[0, j // ps]) * ps + j % ps for j in js]
    inp.q = np.zeros_like(inp.q)
    qpe = np.zeros((1, 16, 64), np.float32)
    for h, r in enumerate(rows):
        kpe = bf16_to_f64(flat[r, 512:])
        qpe[0, h] = np.sign(kpe) * (8000.0 / max(1e-6, np.abs(kpe).sum()))
    inp.q_pe = f32_to_bf16_bits(qpe)
    o, lse, plan = run_decode(torch_cuda, inp, num_cus=cus)
    if cus:
        assert plan.workspace_bytes > 0  # the request is split
    for h, r in enumerate(rows):
        assert np.array_equal(o[0, h], bf16_to_f64(flat[r, :512])), (h, js[h], r)
    ro, _ = oracle(inp)
    assert np.max(np.abs(o - ro)) <= 1e-6  # the fp64 oracle agrees (all weight on one key)


@pytest.mark.parametrize("dt,ps", [("bf16", 64), ("fp8", 64), ("bf16", 16), ("fp8", 16)])
def test_rope_in_its_own_buffer(torch_cuda, dt, ps):
    """The cache's rope columns given through their own base pointer (cache_k_pe, same
    strides as the latent rows), as a cache split into kv_c and k_pe allocations is: the
    rope columns of the main buffer are poisoned (NaN for bf16, 0x7F = NaN for e4m3) and
    must not be read."""
    api = _api()
    torch = torch_cuda
    name = "fp8" if dt == "fp8" else "tiny"
    inp = gen_case(name, seq_lens=np.array([700, 45, 300], np.int32), B=3, N=128, Sq=1, page_size=ps,
                   pool_pages=None, seed=91)
    w = inp.w
    if dt == "bf16":
        cache = bf16_dev(inp.cache)
        poison = torch.full_like(cache[..., 512:], float("nan"))
    else:
        cache = u8_dev(inp.cache)
        poison = torch.full_like(cache[..., 512:], 0x7F)
    pe = torch.zeros_like(cache)  # same shape and strides; only its first 64 columns are rope
    pe[..., :64] = cache[..., 512:]
    cache[..., 512:] = poison
    q, q_pe = bf16_dev(inp.q), bf16_dev(inp.q_pe)
    bt = torch.from_numpy(inp.block_table).to("cuda")
    sl = torch.from_numpy(inp.seq_lens).to("cuda")
    o = torch.full((w.T, w.N, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.T, w.N), float("nan"), dtype=torch.float32, device="cuda")
    kd = api.MLA_DT_BF16 if dt == "bf16" else api.MLA_DT_FP8_E4M3FN
    plan = api.mla_decode_plan(inp.seq_lens, w.Sq, w.N, ps, inp.block_table.shape[1], kd, 0)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    api.mla_decode_run(plan, q, q_pe, cache, bt, sl, w.scale, inp.kv_scale, o, lse, ws, cache_k_pe=pe)
    torch.cuda.synchronize()
    ro, rl = oracle(inp)
    check(bf16_host(o), lse.cpu().numpy().astype(np.float64), ro, rl)


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_one_long_request_split_over_the_chip(torch_cuda, dt):
    """One request of 200,003 keys (ragged last page and tile) with 16 heads: the plan cuts
    it into one segment per compute unit, so the reduce merges a few hundred partial states
    per row (beyond the first batch of partial loads it issues together)."""
    name = "fp8" if dt == "fp8" else "tiny"
    inp = gen_case(name, seq_lens=np.array([200003], np.int32), B=1, N=16, Sq=1, page_size=64,
                   pool_pages=None, seed=23)
    o, lse, plan = run_decode(torch_cuda, inp, num_cus=0)
    work, red = _api().mla_plan_export(plan)
    assert len(work) >= 200 and len(red) == 1
    ro, rl = oracle(inp)
    check(o, lse, ro, rl)
