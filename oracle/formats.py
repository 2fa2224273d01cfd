"""Exact decoding of the storage formats to float64 (oracle; test infrastructure only).

bfloat16: the 16-bit pattern is the upper half of an IEEE float32.
float8 e4m3fn (OCP, the ``torch.float8_e4m3fn`` type that the flashinfer
backend page maps the "fp8" / "fp8_e4m3" cache dtype strings to): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
(value m/8 * 2^-6); 0x7F and 0xFF are NaN; there is no infinity; the largest
finite value is 448.
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to quiet NaN
        return b.view(np.float32).astype(np.float64)


def _e4m3fn_value(byte: int) -> float:
    s = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(i) for i in range(256)], dtype=np.float64)


def e4m3fn_to_f64(bits: np.ndarray) -> np.ndarray:
    return E4M3FN_TABLE[np.asarray(bits, dtype=np.uint8)]


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(bits)
    if dtype == "fp8":
        return e4m3fn_to_f64(bits)
    raise ValueError(dtype)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of each float64 (ties to even), as float64.

    A bfloat16 keeps 8 significant bits: with x = m * 2^e, 0.5 <= |m| < 1, the result is
    round_half_even(m * 2^8) * 2^(e-8).  Values below the normal bfloat16 range, which the
    callers never produce, are not treated specially.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns of round_to_bf16(x) (the upper half of the float32 holding it)."""
    v = round_to_bf16(x).astype(np.float32)
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)

