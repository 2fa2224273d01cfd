"""Static per-tensor fp8 quantisation of the decode query (oracle; test infrastructure only).

Source: vLLM ``layers/attention/mla_attention``, ``MLAAttention`` forward, decode
branch with an fp8 KV cache: when the backend takes a quantised query, ql_nope and
q_pe are concatenated and quantised to float8 e4m3fn with the layer's static
per-tensor ``q_scale`` before the backend call (the ``_DecodeConcatQuantFP8`` op,
static, per-tensor); the ROCm backend then runs with an fp8 query (the
``rocm_aiter_mla`` page: the query dtype is fp8 whenever the cache is fp8).  The
softmax scale picks up q_scale together with the cache scale (the flashinfer page:
``bmm1_scale = scale * q_scale * k_scale``).

The pages do not print the conversion itself.  Reading taken (the usual static
fp8 quantisation): y = float32(x) * float32(1 / q_scale), each operation rounded
to float32, clamped to [-448, 448], then rounded to the nearest e4m3fn value with
ties to the even code.  The e4m3fn grid is the one ``oracle/formats.py`` decodes.

Layout: q8[t, h, 0:512] from ql_nope[t, h, :], q8[t, h, 512:576] from q_pe[t, h, :].
"""
import numpy as np

E4M3_MAX = 448.0


def encode_e4m3fn(y) -> np.ndarray:
    """float32 values with |y| <= 448 -> e4m3fn codes, round to nearest, ties to even.

    Normal range (|y| >= 2^-6): y = 2^e * f with f in [1, 2); the mantissa field is
    (f - 1) * 8 rounded half-to-even; a carry to 8 moves to the next binade.
    Subnormal range: units of 2^-9, rounded half-to-even (8 units = 2^-6 is the
    smallest normal, code 0x08, so the carry needs no special case).
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    if np.any(np.abs(y) > E4M3_MAX) or np.any(np.isnan(y)):
        raise ValueError("encode_e4m3fn takes finite values within +-448")
    sign = np.signbit(y).astype(np.int64) << 7
    a = np.abs(y)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        _, ex = np.frexp(a[nrm])          # a = m * 2^ex, m in [0.5, 1)
        e = ex.astype(np.int64) - 1       # a = f * 2^e, f in [1, 2)
        f = np.ldexp(a[nrm], -e)
        mq = np.rint((f - 1.0) * 8.0).astype(np.int64)
        carry = mq == 8
        e = e + carry
        mq = np.where(carry, 0, mq)
        code[nrm] = ((e + 7) << 3) | mq
    return (code | sign).astype(np.uint8)


def quantize(x_f32, q_scale: float) -> np.ndarray:
    """float32 values -> e4m3fn codes of clamp(x * (1 / q_scale), +-448)."""
    inv = np.float32(1.0) / np.float32(q_scale)
    with np.errstate(over="ignore"):  # a product past the float32 range is +-inf: clamped to +-448
        y = np.asarray(x_f32, dtype=np.float32) * inv
    return encode_e4m3fn(np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX)))


def concat_quant_q(ql_nope_bits, q_pe_bits, q_scale: float) -> np.ndarray:
    """bf16 bit patterns ql_nope [T, N, 512] and q_pe [T, N, 64] -> q8 [T, N, 576] uint8."""
    def f32(bits):
        return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.concatenate([quantize(f32(ql_nope_bits), q_scale), quantize(f32(q_pe_bits), q_scale)], axis=-1)
