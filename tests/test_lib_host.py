"""CPU-side checks of the C-ABI library: exported symbols, the host planner against the
oracle's re-derivation (bit-exact), and argument validation that fails before any HIP call."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

from tests._lib import ROOT, ensure_built

ensure_built()
from mla_paged_decode_03_amd import api  # noqa: E402
from oracle import plan as PL  # noqa: E402


def _header_functions():
    src = open(os.path.join(ROOT, "include", "mla_decode.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _header_functions()
    assert {"mla_decode_plan", "mla_decode_run", "mla_absorb_q", "mla_up_v",
            "merge_attn_states", "mla_plan_destroy", "mla_last_error"} <= set(names)
    out = subprocess.check_output(["nm", "-D", "--defined-only", api.LIB_PATH], text=True)
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(api.exported_symbols()) == set(names)


def _oracle_work(seq_lens, Sq, N, C):
    p = PL.split_plan(seq_lens, Sq, N, C)
    work = np.array(p["items"], dtype=np.int32).reshape(-1, 5)
    red = np.array(p["reduce"], dtype=np.int32).reshape(-1, 3)
    return work, red, p["num_parts"], p["num_partials"]


@pytest.mark.parametrize("seed", range(60))
def test_host_plan_bit_exact_random(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 400))
    L = rng.integers(0, 33000, size=B)
    special = np.array([0, 1, 63, 64, 65, 127, 128, 4096, 32768])
    k = int(rng.integers(0, B + 1))
    L[:k] = rng.choice(special, size=k)
    rng.shuffle(L)
    Sq = int(rng.integers(1, 9))
    N = int(rng.integers(1, 129))
    Cu = int(rng.choice([1, 3, 8, 80, 256, 304]))
    w, r, npart, npartial = api.mla_plan_compute_host(L, Sq, N, Cu)
    ow, orr, onp, onpl = _oracle_work(L, Sq, N, Cu)
    assert np.array_equal(w, ow)
    assert np.array_equal(r, orr)
    assert (npart, npartial) == (onp, onpl)


@pytest.mark.parametrize("name", ["tiny", "dsv3", "longtail", "verify", "fp8"])
def test_host_plan_bit_exact_workloads(name):
    from mla_paged_decode_03_amd import inputs as gen
    w = gen.workload(name)
    rng = np.random.Generator(np.random.PCG64(w.seed))
    L = gen.draw_seq_lens(w, rng)
    got = api.mla_plan_compute_host(L, w.Sq, w.N, 256)
    exp = _oracle_work(L, w.Sq, w.N, 256)
    for a, b in zip(got, exp):
        assert np.array_equal(np.asarray(a), np.asarray(b))


def _plan_rc(**kw):
    args = dict(seq_lens=np.array([10], np.int32), B=1, Sq=1, N=16, Lkv=512, R=64, ps=16, mp=4,
                dt=api.MLA_DT_BF16, cus=1)
    args.update(kw)
    sl = np.ascontiguousarray(args["seq_lens"], dtype=np.int32)
    h = C.c_void_p()
    ws = C.c_size_t()
    rc = api._lib.mla_decode_plan(sl.ctypes.data_as(api._pi32), args["B"], args["Sq"], args["N"],
                                  args["Lkv"], args["R"], args["ps"], args["mp"], args["dt"],
                                  args["cus"], None, C.byref(h), C.byref(ws))
    return rc, api.mla_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(Lkv=256), api.MLA_ERR_UNSUPPORTED),
    (dict(R=32), api.MLA_ERR_UNSUPPORTED),
    (dict(N=129), api.MLA_ERR_UNSUPPORTED),
    (dict(N=0), api.MLA_ERR_UNSUPPORTED),
    (dict(Sq=9), api.MLA_ERR_UNSUPPORTED),
    (dict(Sq=0), api.MLA_ERR_UNSUPPORTED),
    (dict(dt=7), api.MLA_ERR_UNSUPPORTED),
    (dict(B=0), api.MLA_ERR_INVALID_ARG),
    (dict(ps=0), api.MLA_ERR_INVALID_ARG),
    (dict(seq_lens=np.array([65], np.int32)), api.MLA_ERR_INVALID_ARG),  # > 4 pages of 16
    (dict(seq_lens=np.array([-1], np.int32)), api.MLA_ERR_INVALID_ARG),
    (dict(seq_lens=np.array([2 ** 31 - 1], np.int32)), api.MLA_ERR_INVALID_ARG),  # above 2^30 keys
])
def test_plan_argument_errors(kw, code):
    rc, msg = _plan_rc(**kw)
    assert rc == code and msg


def test_null_and_destroy_paths():
    assert api._lib.mla_plan_destroy(None) == api.MLA_OK
    h = C.c_void_p()
    ws = C.c_size_t()
    assert api._lib.mla_decode_plan(None, 1, 1, 16, 512, 64, 16, 4, 0, 1, None, C.byref(h),
                                    C.byref(ws)) == api.MLA_ERR_INVALID_ARG
    rc = api._lib.mla_decode_run(None, None, 0, 0, None, 0, 0, None, None, 0, 0, 0, None, 0, None,
                                 1.0, 1.0, None, 0, 0, None, None, 0, None)
    assert rc == api.MLA_ERR_INVALID_ARG and "plan" in api.mla_last_error()
    assert api._lib.mla_absorb_q(None, None, None, 1, 1, 128, 512, None) == api.MLA_ERR_INVALID_ARG
    assert api._lib.mla_up_v(None, None, None, 1, 1, 512, 128, None) == api.MLA_ERR_INVALID_ARG
    assert api._lib.merge_attn_states(None, None, None, None, None, None, 1, 1, 8, 0, None) == \
        api.MLA_ERR_INVALID_ARG
    assert api._lib.mla_plan_export(None, None, None, None, None) == api.MLA_ERR_INVALID_ARG
    assert api._lib.mla_debug_gather_rows(None, None, 0, None, None) == api.MLA_ERR_INVALID_ARG


def test_gemm_and_merge_shape_errors():
    buf = (C.c_uint8 * 4096)()
    p = C.cast(buf, C.c_void_p).value
    p16 = (p + 15) // 16 * 16
    assert api._lib.mla_absorb_q(p16, p16, p16, 1, 1, 12, 512, None) == api.MLA_ERR_UNSUPPORTED
    assert api._lib.mla_up_v(p16, p16, p16, 1, 1, 512, 12, None) == api.MLA_ERR_UNSUPPORTED
    assert api._lib.merge_attn_states(p16, None, p16, p16, p16, p16, 1, 1, 12, 0, None) == \
        api.MLA_ERR_UNSUPPORTED
    assert api._lib.merge_attn_states(p16, None, p16, p16, p16, p16, 1, 1, 16, 5, None) == \
        api.MLA_ERR_UNSUPPORTED
    assert api._lib.mla_absorb_q(p16 + 2, p16, p16, 1, 1, 128, 512, None) == api.MLA_ERR_INVALID_ARG


def test_concat_quant_argument_errors():
    buf = (C.c_uint8 * 4096)()
    p16 = (C.cast(buf, C.c_void_p).value + 15) // 16 * 16
    q = api._lib.mla_concat_quant_q
    ok = dict(ql=p16, qls=512, qlh=512, qp=p16, qps=64, qph=64, s=1.0, q8=p16, q8s=576, q8h=576, T=1, N=1)

    def call(**kw):
        a = dict(ok, **kw)
        return q(a["ql"], a["qls"], a["qlh"], a["qp"], a["qps"], a["qph"], a["s"], a["q8"], a["q8s"],
                 a["q8h"], a["T"], a["N"], None)
    assert call(ql=None) == api.MLA_ERR_INVALID_ARG
    assert call(q8=None) == api.MLA_ERR_INVALID_ARG
    for s in (0.0, -1.0, float("inf"), float("nan")):
        assert call(s=s) == api.MLA_ERR_INVALID_ARG and "q_scale" in api.mla_last_error()
    assert call(q8h=570) == api.MLA_ERR_INVALID_ARG          # head stride below 576
    assert call(q8h=584, q8s=584) == api.MLA_ERR_INVALID_ARG  # not a multiple of 16
    assert call(ql=p16 + 2) == api.MLA_ERR_INVALID_ARG       # misaligned
    assert call(N=0) == api.MLA_ERR_INVALID_ARG


def test_concat_and_cache_argument_errors():
    buf = (C.c_uint8 * 8192)()
    p16 = (C.cast(buf, C.c_void_p).value + 15) // 16 * 16
    f = api._lib.mla_concat_and_cache
    ok = dict(kv=p16, kvs=512, pe=p16, pes=64, sm=p16, T=1, c=p16, cp=576 * 16, ct=576, ps=16, np_=1,
              dt=api.MLA_DT_BF16, s=1.0)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["kv"], a["kvs"], a["pe"], a["pes"], a["sm"], a["T"], a["c"], a["cp"], a["ct"], a["ps"],
                 a["np_"], a["dt"], a["s"], None)
    assert call(sm=None) == api.MLA_ERR_INVALID_ARG
    assert call(dt=api.MLA_DT_FP32) == api.MLA_ERR_UNSUPPORTED
    assert call(dt=api.MLA_DT_FP8_E4M3FN, s=0.0) == api.MLA_ERR_INVALID_ARG
    assert call(ct=500) == api.MLA_ERR_INVALID_ARG            # token stride below a row
    assert call(cp=576) == api.MLA_ERR_INVALID_ARG            # page stride below a page
    assert call(kv=p16 + 2) == api.MLA_ERR_INVALID_ARG        # misaligned
    assert call(ps=0) == api.MLA_ERR_INVALID_ARG


def _buf16(n=8192):
    buf = (C.c_uint8 * n)()
    return buf, (C.cast(buf, C.c_void_p).value + 255) // 256 * 256


def test_prefill_attention_argument_errors():
    keep, p = _buf16()
    f = api._lib.mla_prefill_attention
    ok = dict(qn=p, qns=128, qnh=128, qp=p, qps=64, qph=64, kn=p, kns=128, knh=128, kp=p, kps=64, v=p, vs=128,
              vh=128, cq=p, ck=p, B=1, mq=1, N=1, P=128, R=64, V=128, causal=1, scale=0.1, o=p, os=128, oh=128)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["qn"], a["qns"], a["qnh"], a["qp"], a["qps"], a["qph"], a["kn"], a["kns"], a["knh"], a["kp"],
                 a["kps"], a["v"], a["vs"], a["vh"], a["cq"], a["ck"], a["B"], a["mq"], a["N"], a["P"], a["R"],
                 a["V"], a["causal"], a["scale"], a["o"], a["os"], a["oh"], None, None)
    assert call(cq=None) == api.MLA_ERR_INVALID_ARG
    assert call(P=64) == api.MLA_ERR_UNSUPPORTED and call(V=64) == api.MLA_ERR_UNSUPPORTED
    for s in (0.0, -1.0, float("nan"), float("inf")):
        assert call(scale=s) == api.MLA_ERR_INVALID_ARG
    assert call(vh=120) == api.MLA_ERR_INVALID_ARG       # head stride below V
    assert call(kps=60) == api.MLA_ERR_INVALID_ARG       # rope row shorter than R
    assert call(os=132, oh=132) == api.MLA_ERR_INVALID_ARG  # not 16-byte rows
    assert call(o=p + 2) == api.MLA_ERR_INVALID_ARG
    assert call(N=0) == api.MLA_ERR_INVALID_ARG
    assert call(vs=1 << 25, kns=1 << 25) == api.MLA_ERR_UNSUPPORTED  # 32-bit tile row offsets


def test_gather_and_kv_b_proj_argument_errors():
    keep, p = _buf16()
    g = api._lib.mla_gather_context
    ok = dict(c=p, pe=p, sp=576 * 16, st=576, ps=16, dt=api.MLA_DT_BF16, s=1.0, bt=p, bts=4, starts=p, cu=p, B=1,
              tot=1, okv=p, okvs=512, ope=p, opes=64)

    def call(**kw):
        a = dict(ok, **kw)
        return g(a["c"], a["pe"], a["sp"], a["st"], a["ps"], a["dt"], a["s"], a["bt"], a["bts"], a["starts"],
                 a["cu"], a["B"], a["tot"], a["okv"], a["okvs"], a["ope"], a["opes"], None)
    assert call(cu=None) == api.MLA_ERR_INVALID_ARG
    assert call(dt=api.MLA_DT_FP32) == api.MLA_ERR_UNSUPPORTED
    assert call(dt=api.MLA_DT_FP8_E4M3FN, s=0.0) == api.MLA_ERR_INVALID_ARG
    assert call(st=500) == api.MLA_ERR_INVALID_ARG and call(okvs=500) == api.MLA_ERR_INVALID_ARG
    assert call(okv=p + 2) == api.MLA_ERR_INVALID_ARG
    k = api._lib.mla_kv_b_proj
    assert k(p, 512, p, p, p, p, 4, 2, 512, 12, 128, None) == api.MLA_ERR_UNSUPPORTED
    assert k(p, 100, p, p, p, p, 4, 2, 512, 128, 128, None) == api.MLA_ERR_INVALID_ARG
    assert k(None, 512, p, p, p, p, 4, 2, 512, 128, 128, None) == api.MLA_ERR_INVALID_ARG


def test_chunked_prefill_workspace_size_and_errors():
    # the chunk schedule: with k requests that have context, mcc = workspace_tokens / k
    # rounded down to the page size; mcc = 0 is a workspace error
    with pytest.raises(api.MLAError) as e:
        api.mla_chunked_prefill_workspace_size([1, 1, 1], [5, 5, 5], 8, 128, 128, 16, 2)
    assert e.value.status == api.MLA_ERR_WORKSPACE
    no_ctx = api.mla_chunked_prefill_workspace_size([7, 9], [0, 0], 8, 128, 128, 16, 64)
    ctx = api.mla_chunked_prefill_workspace_size([7, 9], [100, 0], 8, 128, 128, 16, 64)
    more = api.mla_chunked_prefill_workspace_size([70, 90], [100, 0], 8, 128, 128, 16, 64)
    assert 0 < no_ctx < ctx < more
    # the k_nope / v buffers cover the larger of the new tokens and the largest chunk
    small = api.mla_chunked_prefill_workspace_size([1], [64], 8, 128, 128, 16, 64)
    big = api.mla_chunked_prefill_workspace_size([1], [64], 8, 128, 128, 16, 128)
    assert big == small  # one chunk of 64 either way
    keep, p = _buf16()
    f = api._lib.mla_chunked_prefill
    nl = np.array([2], np.int32)
    cl = np.array([0], np.int32)
    pi = nl.ctypes.data_as(C.POINTER(C.c_int32))
    pc = cl.ctypes.data_as(C.POINTER(C.c_int32))
    args = [p, p, p, p, pi, pc, 1, p, p, 576 * 16, 576, 16, 0, 1.0, p, 4, p, p, 2, 512, 128, 64, 128, 0.1, 64, p,
            None, p, 1 << 20, None]
    a = list(args)
    a[0] = None
    assert f(*a) == api.MLA_ERR_INVALID_ARG
    a = list(args)
    a[20] = 64  # P
    assert f(*a) == api.MLA_ERR_UNSUPPORTED


def test_fp8_bmm_argument_errors():
    keep, p = _buf16()
    q = api._lib.mla_quant_weight_fp8
    assert q(p, 512, 2, 128, 2, p, p, None) == api.MLA_ERR_INVALID_ARG   # which
    assert q(p, 512, 2, 12, 0, p, p, None) == api.MLA_ERR_INVALID_ARG    # X not a multiple of 8
    assert q(p + 2, 512, 2, 128, 0, p, p, None) == api.MLA_ERR_INVALID_ARG
    a = api._lib.mla_absorb_q_fp8
    assert a(p, p, None, p, 1, 2, 128, 512, None) == api.MLA_ERR_INVALID_ARG  # w_scale
    assert a(p, p, p, p, 1, 2, 192, 512, None) == api.MLA_ERR_UNSUPPORTED    # P not a multiple of 128
    u = api._lib.mla_up_v_fp8
    assert u(p, p, p, p, 1, 2, 500, 128, None) == api.MLA_ERR_UNSUPPORTED    # Lkv not a multiple of 128
    assert u(p, p, p, p, 1, 2, 512, 12, None) == api.MLA_ERR_UNSUPPORTED     # V not a multiple of 8


def test_plan_compute_host_rejects_overflowing_seq_len():
    """seq_len + 63 (the granule round-up) must not wrap: lengths above 2^30 are rejected."""
    n_items, n_red = C.c_int32(0), C.c_int32(0)
    for L in (2 ** 31 - 1, 2 ** 31 - 64, 2 ** 30 + 1):
        sl = np.array([5, L], np.int32)
        rc = api._lib.mla_plan_compute_host(sl.ctypes.data_as(C.POINTER(C.c_int32)), 2, 1, 128, 256, None,
                                            C.byref(n_items), None, C.byref(n_red), None, None)
        assert rc == api.MLA_ERR_INVALID_ARG and "seq_len" in api.mla_last_error()
    sl = np.array([2 ** 30], np.int32)  # the largest accepted length plans normally
    rc = api._lib.mla_plan_compute_host(sl.ctypes.data_as(C.POINTER(C.c_int32)), 1, 1, 128, 256, None,
                                        C.byref(n_items), None, C.byref(n_red), None, None)
    assert rc == api.MLA_OK and n_items.value == 256 and n_red.value == 1
