"""ctypes binding of libmla_decode.so: the C ABI of include/mla_decode.h, same names.

Argument marshalling only: every step of the decode runs in the HIP library.
torch supplies device memory and the current stream.  If the library has not
been built this module raises on import, so no caller can fall back to
anything else.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_decode.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP, MLA_ERR_INTERNAL = \
    0, -1, -2, -3, -4, -5
MLA_DT_BF16, MLA_DT_FP8_E4M3FN, MLA_DT_FP32 = 0, 1, 2
LKV, ROPE = 512, 64

# torch first: it loads its own HIP runtime (SONAME libamdhip64.so.7), which the
# library's dependency then resolves to, so the process holds exactly one runtime
# and the library shares torch's devices, streams and allocations.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mla_paged_decode_03_amd.build`")
_lib = C.CDLL(LIB_PATH)

_i32, _i64, _f32, _vp, _sz = C.c_int32, C.c_int64, C.c_float, C.c_void_p, C.c_size_t
_pi32, _pi64, _pf32 = C.POINTER(C.c_int32), C.POINTER(C.c_int64), C.POINTER(C.c_float)

_SIGS = {
    "mla_decode_plan": [_pi32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp,
                        C.POINTER(_vp), C.POINTER(_sz)],
    "mla_plan_destroy": [_vp],
    "mla_decode_run": [_vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _i32, _vp, _i64,
                       _vp, _f32, _f32, _vp, _i64, _i64, _vp, _vp, _sz, _vp],
    "mla_decode_run_noalloc": [_vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _i32, _vp, _i64,
                               _vp, _f32, _f32, _vp, _i64, _i64, _vp, _vp],
    "mla_decode_attend": [_vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _i32, _vp,
                          _i64, _vp, _f32, _f32, _vp, _i64, _i64, _vp, _vp, _sz, _vp],
    "mla_decode_reduce": [_vp, _vp, _i64, _i64, _vp, _vp, _sz, _vp],
    "mla_absorb_q": [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp],
    "mla_up_v": [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp],
    "merge_attn_states": [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp],
    "mla_last_error": [],
    "mla_plan_compute_host": [_pi32, _i32, _i32, _i32, _i32, _pi32, _pi32, _pi32, _pi32, _pi32, _pi32],
    "mla_plan_export": [_vp, _pi32, _pi32, _pi32, _pi32],
    "mla_debug_gather_rows": [_vp, _vp, _i64, _vp, _vp],
    "mla_concat_quant_q": [_vp, _i64, _i64, _vp, _i64, _i64, _f32, _vp, _i64, _i64, _i32, _i32, _vp],
    "mla_concat_and_cache": [_vp, _i64, _vp, _i64, _vp, _i32, _vp, _i64, _i64, _i32, _i32, _i32, _f32, _vp],
    "mla_decode_run_q8": [_vp, _vp, _i64, _i64, _f32, _vp, _vp, _i64, _i64, _i32, _vp, _i64, _vp, _f32, _f32,
                          _vp, _i64, _i64, _vp, _vp, _sz, _vp],
    "mla_decode_attend_q8": [_vp, _vp, _i64, _i64, _f32, _vp, _vp, _i64, _i64, _i32, _vp, _i64, _vp, _f32,
                             _f32, _vp, _i64, _i64, _vp, _vp, _sz, _vp],
    "mla_prefill_attention": [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64,
                              _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _i64, _i64, _vp,
                              _vp],
    "mla_gather_context": [_vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp, _i64, _vp, _vp, _i32, _i64, _vp, _i64,
                           _vp, _i64, _vp],
    "mla_kv_b_proj": [_vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp],
    "mla_quant_weight_fp8": [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp],
    "mla_absorb_q_fp8": [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp],
    "mla_up_v_fp8": [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp],
    "mla_chunked_prefill_workspace_size": [_pi32, _pi32, _i32, _i32, _i32, _i32, _i32, _i64, C.POINTER(_sz)],
    "mla_chunked_prefill": [_vp, _vp, _vp, _vp, _pi32, _pi32, _i32, _vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp,
                            _i64, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _i64, _vp, _vp, _vp, _sz, _vp],
}
for _name, _args in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = C.c_char_p if _name == "mla_last_error" else C.c_int


class MLAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def mla_last_error() -> str:
    return _lib.mla_last_error().decode()


def _check(rc: int):
    if rc != MLA_OK:
        raise MLAError(rc, mla_last_error())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _host_i32(x) -> np.ndarray:
    if hasattr(x, "cpu"):
        x = x.cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


@dataclass
class Plan:
    handle: int
    workspace_bytes: int
    B: int
    Sq: int
    N: int
    page_size: int
    max_pages: int
    kv_dtype: int

    def destroy(self):
        if self.handle:
            _check(_lib.mla_plan_destroy(self.handle))
            self.handle = 0

    def __del__(self):
        try:
            if self.handle:
                _lib.mla_plan_destroy(self.handle)
        except Exception:
            pass


def mla_decode_plan(seq_lens, Sq: int, N: int, page_size: int, max_pages_per_req: int,
                    kv_dtype: int = MLA_DT_BF16, num_cus: int = 0, stream=None,
                    Lkv: int = LKV, R: int = ROPE) -> Plan:
    sl = _host_i32(seq_lens)
    h = _vp()
    ws = _sz()
    _check(_lib.mla_decode_plan(sl.ctypes.data_as(_pi32), len(sl), Sq, N, Lkv, R, page_size,
                                max_pages_per_req, kv_dtype, num_cus, _stream(stream),
                                C.byref(h), C.byref(ws)))
    return Plan(h.value, ws.value, len(sl), Sq, N, page_size, max_pages_per_req, kv_dtype)


def mla_plan_destroy(plan: Plan):
    plan.destroy()


def _need(t, dtypes, name):
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")


def _decode_args(plan: Plan, q_nope, q_pe, cache, block_table, seq_lens, scale, kv_scale,
                 o_latent, lse, workspace, stream, cache_k_pe):
    bf, f8 = torch.bfloat16, (torch.float8_e4m3fn, torch.uint8)
    _need(q_nope, (bf,), "q_nope")
    _need(q_pe, (bf,), "q_pe")
    _need(cache, (bf,) if plan.kv_dtype == MLA_DT_BF16 else f8, "cache")
    _need(block_table, (torch.int32,), "block_table")
    _need(seq_lens, (torch.int32,), "seq_lens")
    _need(o_latent, (bf,), "o_latent")
    if lse is not None:
        _need(lse, (torch.float32,), "lse")
        if not lse.is_contiguous():
            raise ValueError("lse must be contiguous [T, N]")
    if q_nope.stride(2) != 1 or q_pe.stride(2) != 1 or o_latent.stride(2) != 1 or cache.stride(2) != 1:
        raise ValueError("the last dimension of every tensor must be contiguous")
    esz = cache.element_size()
    kpe_ptr = cache.data_ptr() + LKV * esz if cache_k_pe is None else cache_k_pe.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (plan.handle, q_nope.data_ptr(), q_nope.stride(0), q_nope.stride(1),
            q_pe.data_ptr(), q_pe.stride(0), q_pe.stride(1),
            cache.data_ptr(), kpe_ptr, cache.stride(0), cache.stride(1), cache.shape[0],
            block_table.data_ptr(), block_table.stride(0), seq_lens.data_ptr(),
            float(scale), float(kv_scale), o_latent.data_ptr(), o_latent.stride(0),
            o_latent.stride(1), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream))


def mla_decode_run(plan: Plan, q_nope, q_pe, cache, block_table, seq_lens, scale: float,
                   kv_scale: float, o_latent, lse=None, workspace=None, stream=None,
                   cache_k_pe=None):
    """q_nope [T,N,512] bf16, q_pe [T,N,64] bf16, cache [pages, page_size, 576] (bf16 or fp8;
    or the kv_c part when cache_k_pe is given), block_table [B, max_pages] int32,
    seq_lens [B] int32 (device), o_latent [T,N,512] bf16, lse [T,N] fp32 or None."""
    _check(_lib.mla_decode_run(*_decode_args(plan, q_nope, q_pe, cache, block_table, seq_lens, scale,
                                             kv_scale, o_latent, lse, workspace, stream, cache_k_pe)))


def mla_decode_run_noalloc(plan: Plan, q_nope, q_pe, cache, block_table, seq_lens, scale: float,
                           kv_scale: float, o_latent, lse=None, stream=None, cache_k_pe=None):
    """mla_decode_run with the library's static device scratch as the workspace (no
    allocation; plans needing more than 64 MiB of workspace are rejected)."""
    args = _decode_args(plan, q_nope, q_pe, cache, block_table, seq_lens, scale, kv_scale, o_latent, lse,
                        None, stream, cache_k_pe)
    _check(_lib.mla_decode_run_noalloc(*(args[:21] + args[23:])))


def mla_decode_attend(plan: Plan, q_nope, q_pe, cache, block_table, seq_lens, scale: float,
                      kv_scale: float, o_latent, lse=None, workspace=None, stream=None,
                      cache_k_pe=None):
    """First phase of mla_decode_run (the decode kernel); same arguments."""
    _check(_lib.mla_decode_attend(*_decode_args(plan, q_nope, q_pe, cache, block_table, seq_lens,
                                                scale, kv_scale, o_latent, lse, workspace, stream,
                                                cache_k_pe)))


def _decode_args_q8(plan: Plan, q8, q_scale, cache, block_table, seq_lens, scale, kv_scale,
                    o_latent, lse, workspace, stream, cache_k_pe):
    _need(q8, (torch.float8_e4m3fn, torch.uint8), "q8")
    if q8.stride(2) != 1:
        raise ValueError("the last dimension of q8 must be contiguous")
    # the bf16 argument checks, with the fp8 query standing in for q_nope / q_pe
    args = list(_decode_args(plan, o_latent, o_latent, cache, block_table, seq_lens, scale, kv_scale,
                             o_latent, lse, workspace, stream, cache_k_pe))
    return (args[0], q8.data_ptr(), q8.stride(0), q8.stride(1), float(q_scale)) + tuple(args[7:])


def mla_decode_run_q8(plan: Plan, q8, q_scale: float, cache, block_table, seq_lens, scale: float,
                      kv_scale: float, o_latent, lse=None, workspace=None, stream=None, cache_k_pe=None):
    """q8 [T,N,576] float8_e4m3fn ([ql_nope | q_pe] quantised with q_scale, see
    mla_concat_quant_q); the cache must be fp8.  Other arguments as mla_decode_run."""
    _check(_lib.mla_decode_run_q8(*_decode_args_q8(plan, q8, q_scale, cache, block_table, seq_lens, scale,
                                                   kv_scale, o_latent, lse, workspace, stream, cache_k_pe)))


def mla_decode_attend_q8(plan: Plan, q8, q_scale: float, cache, block_table, seq_lens, scale: float,
                         kv_scale: float, o_latent, lse=None, workspace=None, stream=None, cache_k_pe=None):
    """First phase of mla_decode_run_q8; same arguments."""
    _check(_lib.mla_decode_attend_q8(*_decode_args_q8(plan, q8, q_scale, cache, block_table, seq_lens,
                                                      scale, kv_scale, o_latent, lse, workspace, stream,
                                                      cache_k_pe)))


def mla_decode_reduce(plan: Plan, o_latent, lse=None, workspace=None, stream=None):
    """Second phase of mla_decode_run: merges the partial states of split requests."""
    _need(o_latent, (torch.bfloat16,), "o_latent")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.mla_decode_reduce(plan.handle, o_latent.data_ptr(), o_latent.stride(0),
                                  o_latent.stride(1), _ptr(lse), _ptr(workspace), ws_bytes,
                                  _stream(stream)))


def _need_contig_bf16(*ts):
    for t in ts:
        _need(t, (torch.bfloat16,), "tensor")
        if not t.is_contiguous():
            raise ValueError("absorb / up-projection tensors must be contiguous")


def mla_absorb_q(q_nope, W_UK, ql_nope, stream=None):
    _need_contig_bf16(q_nope, W_UK, ql_nope)
    T, N, P = q_nope.shape
    Lkv = W_UK.shape[0]
    _check(_lib.mla_absorb_q(q_nope.data_ptr(), W_UK.data_ptr(), ql_nope.data_ptr(), T, N, P, Lkv,
                             _stream(stream)))


def mla_up_v(o_latent, W_UV, o, stream=None):
    _need_contig_bf16(o_latent, W_UV, o)
    T, N, Lkv = o_latent.shape
    V = W_UV.shape[2]
    _check(_lib.mla_up_v(o_latent.data_ptr(), W_UV.data_ptr(), o.data_ptr(), T, N, Lkv, V,
                         _stream(stream)))


def merge_attn_states(out, out_lse, prefix_o, prefix_lse, suffix_o, suffix_lse, stream=None):
    T, N, D = out.shape
    for t in (out, prefix_o, suffix_o):
        _need(t, (out.dtype,), "merge state")
        if not t.is_contiguous():
            raise ValueError("merge states must be contiguous [T, N, D]")
    for t in (prefix_lse, suffix_lse) + ((out_lse,) if out_lse is not None else ()):
        _need(t, (torch.float32,), "lse")
    dt = MLA_DT_FP32 if out.dtype == torch.float32 else MLA_DT_BF16
    _check(_lib.merge_attn_states(out.data_ptr(), _ptr(out_lse), prefix_o.data_ptr(),
                                  prefix_lse.data_ptr(), suffix_o.data_ptr(), suffix_lse.data_ptr(),
                                  T, N, D, dt, _stream(stream)))


def mla_concat_quant_q(ql_nope, q_pe, q_scale: float, q8, stream=None):
    """ql_nope [T,N,512] bf16, q_pe [T,N,64] bf16 -> q8 [T,N,576] float8_e4m3fn (or uint8)."""
    _need(ql_nope, (torch.bfloat16,), "ql_nope")
    _need(q_pe, (torch.bfloat16,), "q_pe")
    _need(q8, (torch.float8_e4m3fn, torch.uint8), "q8")
    T, N, _ = ql_nope.shape
    if tuple(q_pe.shape) != (T, N, ROPE) or tuple(q8.shape) != (T, N, LKV + ROPE) or ql_nope.shape[2] != LKV:
        raise ValueError("shapes must be ql_nope [T,N,512], q_pe [T,N,64], q8 [T,N,576]")
    for t in (ql_nope, q_pe, q8):
        if t.stride(2) != 1:
            raise ValueError("the last dimension must be contiguous")
    _check(_lib.mla_concat_quant_q(ql_nope.data_ptr(), ql_nope.stride(0), ql_nope.stride(1),
                                   q_pe.data_ptr(), q_pe.stride(0), q_pe.stride(1), float(q_scale),
                                   q8.data_ptr(), q8.stride(0), q8.stride(1), T, N, _stream(stream)))


def mla_concat_and_cache(kv_c, k_pe, slot_mapping, cache, k_scale: float = 1.0, stream=None):
    """kv_c [T,512] bf16, k_pe [T,64] bf16, slot_mapping [T] int64 (device), cache
    [num_pages, page_size, 576] bf16 or float8_e4m3fn / uint8 (fp8: quantised with k_scale)."""
    _need(kv_c, (torch.bfloat16,), "kv_c")
    _need(k_pe, (torch.bfloat16,), "k_pe")
    _need(slot_mapping, (torch.int64,), "slot_mapping")
    _need(cache, (torch.bfloat16, torch.float8_e4m3fn, torch.uint8), "cache")
    T = kv_c.shape[0]
    if tuple(kv_c.shape) != (T, LKV) or tuple(k_pe.shape) != (T, ROPE) or tuple(slot_mapping.shape) != (T,):
        raise ValueError("shapes must be kv_c [T,512], k_pe [T,64], slot_mapping [T]")
    if cache.dim() != 3 or cache.shape[2] != LKV + ROPE or cache.stride(2) != 1:
        raise ValueError("cache must be [num_pages, page_size, 576] with contiguous rows")
    if kv_c.stride(1) != 1 or k_pe.stride(1) != 1 or not slot_mapping.is_contiguous():
        raise ValueError("the last dimension must be contiguous")
    dt = MLA_DT_BF16 if cache.dtype == torch.bfloat16 else MLA_DT_FP8_E4M3FN
    _check(_lib.mla_concat_and_cache(kv_c.data_ptr(), kv_c.stride(0), k_pe.data_ptr(), k_pe.stride(0),
                                     slot_mapping.data_ptr(), T, cache.data_ptr(), cache.stride(0),
                                     cache.stride(1), cache.shape[1], cache.shape[0], dt, float(k_scale),
                                     _stream(stream)))


def mla_plan_compute_host(seq_lens, Sq: int, N: int, num_cus: int):
    """Host-only plan rule: (work [n,5] int32, reduce [m,3] int32, num_parts, num_partials)."""
    sl = _host_i32(seq_lens)
    ni, nr, npart, npartial = _i32(0), _i32(0), _i32(0), _i32(0)
    _check(_lib.mla_plan_compute_host(sl.ctypes.data_as(_pi32), len(sl), Sq, N, num_cus, None,
                                      C.byref(ni), None, C.byref(nr), C.byref(npart), C.byref(npartial)))
    work = np.zeros((max(ni.value, 1), 5), dtype=np.int32)
    red = np.zeros((max(nr.value, 1), 3), dtype=np.int32)
    _check(_lib.mla_plan_compute_host(sl.ctypes.data_as(_pi32), len(sl), Sq, N, num_cus,
                                      work.ctypes.data_as(_pi32), C.byref(ni),
                                      red.ctypes.data_as(_pi32), C.byref(nr), C.byref(npart),
                                      C.byref(npartial)))
    return work[:ni.value], red[:nr.value], npart.value, npartial.value


def mla_plan_export(plan: Plan):
    ni, nr = _i32(0), _i32(0)
    _check(_lib.mla_plan_export(plan.handle, None, C.byref(ni), None, C.byref(nr)))
    work = np.zeros((max(ni.value, 1), 5), dtype=np.int32)
    red = np.zeros((max(nr.value, 1), 3), dtype=np.int32)
    _check(_lib.mla_plan_export(plan.handle, work.ctypes.data_as(_pi32), C.byref(ni),
                                red.ctypes.data_as(_pi32), C.byref(nr)))
    return work[:ni.value], red[:nr.value]


def mla_debug_gather_rows(plan: Plan, block_table, rows_out, stream=None):
    _need(block_table, (torch.int32,), "block_table")
    _need(rows_out, (torch.int64,), "rows_out")
    _check(_lib.mla_debug_gather_rows(plan.handle, block_table.data_ptr(), block_table.stride(0),
                                      rows_out.data_ptr(), _stream(stream)))


def _rows16(t, name):
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")


def mla_prefill_attention(q_nope, q_pe, k_nope, k_pe, v, cu_q, cu_k, max_q: int, causal: bool,
                          scale: float, o, lse=None, stream=None):
    """Per-head attention of the compute-friendly path: q_nope [T,N,128], q_pe [T,N,64],
    k_nope [S,N,128], k_pe [S,64] (shared by the heads), v [S,N,128] bf16; cu_q / cu_k
    [B+1] int32 device offsets of each request's queries and keys; o [T,N,128] bf16,
    lse [T,N] fp32 or None."""
    for t, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (k_nope, "k_nope"), (k_pe, "k_pe"), (v, "v"), (o, "o")):
        _need(t, (torch.bfloat16,), n)
        _rows16(t, n)
    for t, n in ((cu_q, "cu_q"), (cu_k, "cu_k")):
        _need(t, (torch.int32,), n)
    if lse is not None:
        _need(lse, (torch.float32,), "lse")
        if not lse.is_contiguous():
            raise ValueError("lse must be contiguous [T, N]")
    T, N, P = q_nope.shape
    B = cu_q.shape[0] - 1
    _check(_lib.mla_prefill_attention(
        q_nope.data_ptr(), q_nope.stride(0), q_nope.stride(1), q_pe.data_ptr(), q_pe.stride(0), q_pe.stride(1),
        k_nope.data_ptr(), k_nope.stride(0), k_nope.stride(1), k_pe.data_ptr(), k_pe.stride(0),
        v.data_ptr(), v.stride(0), v.stride(1), cu_q.data_ptr(), cu_k.data_ptr(), B, int(max_q), N, P,
        q_pe.shape[2], v.shape[2], int(bool(causal)), float(scale), o.data_ptr(), o.stride(0), o.stride(1),
        _ptr(lse), _stream(stream)))


def mla_gather_context(cache, block_table, starts, cu, total: int, out_kv_c, out_k_pe,
                       kv_scale: float = 1.0, stream=None):
    """Rows of one context chunk: out row r of request b (cu[b] <= r < cu[b+1]) is the
    cache row of position starts[b] + r - cu[b]; bf16 out_kv_c [n,512], out_k_pe [n,64]."""
    _need(cache, (torch.bfloat16, torch.float8_e4m3fn, torch.uint8), "cache")
    for t, n in ((block_table, "block_table"), (starts, "starts"), (cu, "cu")):
        _need(t, (torch.int32,), n)
    _need(out_kv_c, (torch.bfloat16,), "out_kv_c")
    _need(out_k_pe, (torch.bfloat16,), "out_k_pe")
    if cache.dim() != 3 or cache.shape[2] != LKV + ROPE or cache.stride(2) != 1:
        raise ValueError("cache must be [num_pages, page_size, 576] with contiguous rows")
    dt = MLA_DT_BF16 if cache.dtype == torch.bfloat16 else MLA_DT_FP8_E4M3FN
    kpe = cache.data_ptr() + LKV * cache.element_size()
    _check(_lib.mla_gather_context(cache.data_ptr(), kpe, cache.stride(0), cache.stride(1), cache.shape[1], dt,
                                   float(kv_scale), block_table.data_ptr(), block_table.stride(0),
                                   starts.data_ptr(), cu.data_ptr(), starts.shape[0], int(total),
                                   out_kv_c.data_ptr(), out_kv_c.stride(0), out_k_pe.data_ptr(),
                                   out_k_pe.stride(0), _stream(stream)))


def mla_kv_b_proj(kv_c, W_UK, W_UV, k_nope, v, stream=None):
    """k_nope[s,h,:] = kv_c[s] . W_UK[:,h,:], v[s,h,:] = kv_c[s] . W_UV[:,h,:] (bf16)."""
    _need_contig_bf16(W_UK, W_UV, k_nope, v)
    _need(kv_c, (torch.bfloat16,), "kv_c")
    _rows16(kv_c, "kv_c")
    S, Lkv = kv_c.shape
    _, N, P = W_UK.shape
    V = W_UV.shape[2]
    _check(_lib.mla_kv_b_proj(kv_c.data_ptr(), kv_c.stride(0), W_UK.data_ptr(), W_UV.data_ptr(),
                              k_nope.data_ptr(), v.data_ptr(), S, N, Lkv, P, V, _stream(stream)))


def mla_chunked_prefill_workspace_size(new_lens, ctx_lens, N: int, P: int, V: int, page_size: int,
                                       workspace_tokens: int) -> int:
    nl, cl = _host_i32(new_lens), _host_i32(ctx_lens)
    out = _sz(0)
    _check(_lib.mla_chunked_prefill_workspace_size(nl.ctypes.data_as(_pi32), cl.ctypes.data_as(_pi32), len(nl),
                                                   N, P, V, page_size, int(workspace_tokens), C.byref(out)))
    return out.value


def mla_chunked_prefill(q_nope, q_pe, kv_c, k_pe, new_lens, ctx_lens, cache, block_table, W_UK, W_UV,
                        scale: float, workspace_tokens: int, o, lse=None, workspace=None, kv_scale: float = 1.0,
                        stream=None):
    """Chunked prefill of a batch (compute-friendly form): new tokens q_nope [T,N,128],
    q_pe [T,N,64], their latent rows kv_c [T,512] and k_pe [T,64] (contiguous bf16);
    new_lens / ctx_lens [B] host counts; context in the paged cache through block_table;
    W_UK / W_UV [512,N,128]; o [T,N,128] bf16, lse [T,N] fp32 or None."""
    _need_contig_bf16(q_nope, q_pe, kv_c, k_pe, W_UK, W_UV, o)
    _need(cache, (torch.bfloat16, torch.float8_e4m3fn, torch.uint8), "cache")
    _need(block_table, (torch.int32,), "block_table")
    if lse is not None:
        _need(lse, (torch.float32,), "lse")
        if not lse.is_contiguous():
            raise ValueError("lse must be contiguous [T, N]")
    nl, cl = _host_i32(new_lens), _host_i32(ctx_lens)
    T, N, P = q_nope.shape
    V = W_UV.shape[2]
    dt = MLA_DT_BF16 if cache.dtype == torch.bfloat16 else MLA_DT_FP8_E4M3FN
    kpe = cache.data_ptr() + LKV * cache.element_size()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.mla_chunked_prefill(
        q_nope.data_ptr(), q_pe.data_ptr(), kv_c.data_ptr(), k_pe.data_ptr(), nl.ctypes.data_as(_pi32),
        cl.ctypes.data_as(_pi32), len(nl), cache.data_ptr(), kpe, cache.stride(0), cache.stride(1),
        cache.shape[1], dt, float(kv_scale), block_table.data_ptr(), block_table.stride(0), W_UK.data_ptr(),
        W_UV.data_ptr(), N, W_UK.shape[0], P, q_pe.shape[2], V, float(scale), int(workspace_tokens),
        o.data_ptr(), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def mla_quant_weight_fp8(W, which: str, W8, w_scale, stream=None):
    """W_UK [Lkv,N,P] (which "uk") -> W_K [N,Lkv,P], or W_UV [Lkv,N,V] ("uv") -> W_V [N,V,Lkv],
    e4m3fn (float8_e4m3fn or uint8 tensor W8); w_scale: device float32 [1]."""
    _need_contig_bf16(W)
    _need(W8, (torch.float8_e4m3fn, torch.uint8), "W8")
    _need(w_scale, (torch.float32,), "w_scale")
    Lkv, N, X = W.shape
    want = (N, Lkv, X) if which == "uk" else (N, X, Lkv)
    if tuple(W8.shape) != want or not W8.is_contiguous():
        raise ValueError(f"W8 must be contiguous {want}")
    _check(_lib.mla_quant_weight_fp8(W.data_ptr(), Lkv, N, X, 0 if which == "uk" else 1, W8.data_ptr(),
                                     w_scale.data_ptr(), _stream(stream)))


def mla_absorb_q_fp8(q_nope, W_K, w_scale, ql_nope, stream=None):
    """ql_nope [T,N,Lkv] = fp8 BMM of q_nope [T,N,P] with W_K [N,Lkv,P] (e4m3fn) and w_scale."""
    _need_contig_bf16(q_nope, ql_nope)
    _need(W_K, (torch.float8_e4m3fn, torch.uint8), "W_K")
    _need(w_scale, (torch.float32,), "w_scale")
    T, N, P = q_nope.shape
    Lkv = W_K.shape[1]
    _check(_lib.mla_absorb_q_fp8(q_nope.data_ptr(), W_K.data_ptr(), w_scale.data_ptr(), ql_nope.data_ptr(),
                                 T, N, P, Lkv, _stream(stream)))


def mla_up_v_fp8(o_latent, W_V, w_scale, o, stream=None):
    """o [T,N,V] = fp8 BMM of o_latent [T,N,Lkv] with W_V [N,V,Lkv] (e4m3fn) and w_scale."""
    _need_contig_bf16(o_latent, o)
    _need(W_V, (torch.float8_e4m3fn, torch.uint8), "W_V")
    _need(w_scale, (torch.float32,), "w_scale")
    T, N, Lkv = o_latent.shape
    V = W_V.shape[1]
    _check(_lib.mla_up_v_fp8(o_latent.data_ptr(), W_V.data_ptr(), w_scale.data_ptr(), o.data_ptr(),
                             T, N, Lkv, V, _stream(stream)))


def exported_symbols():
    return list(_SIGS)
