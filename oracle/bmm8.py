"""fp8 batched GEMMs for the W_UK absorption and the W_UV up-projection (oracle; test
infrastructure only).

Source: vLLM ``v1/attention/backends/mla/common.py`` and ``layers/attention/
mla_attention``, ``process_weights_after_loading`` with the ROCm fp8 BMM enabled:
the weights are laid out per head, W_K = W_UK transposed to [N, Lkv, P] and
W_V = W_UV permuted to [N, V, Lkv], and each is quantised to float8 e4m3fn with one
scale for the whole tensor (``dynamic_per_batched_tensor_quant``); the absorption
(``_forward_decode`` / ``forward_mqa`` path) and ``_v_up_proj`` then call a batched
GEMM whose activations are quantised per token in groups of 128 along the contracted
dimension ("a8w8, a per token group prequant, w per batched tensor quant", group_size
128).

Weight quantisation, as the page computes it on bf16 tensors (every bf16 operation is
done in float32 and rounded to bf16, ties to even): amax = max |W| (at least 1e-10),
s = bf16(448 / amax), y = bf16(W * s), clamped to +-448, code = e4m3fn(y) rounded to
nearest even; the dequantisation scale is float32(1 / s).

Activation quantisation (the pages name it, but print no arithmetic; reading taken:
the weights' formula per group, in float32; parity unpinned: no printed value or
reference implementation fixes it, only the quantisation invariants of the tests):
for token m and group g of 128 consecutive contracted elements,
amax = max |a| (at least 1e-10), s = float32(448 / amax),
y = float32(a * s) clamped to +-448, code = e4m3fn(y); dequantisation d = float32(1 / s).

Product: C[h, m, n] = w_scale * sum_g d[h, m, g] * sum_{k in g} A8[h, m, k] W8[h, n, k],
with the codes decoded exactly (float64).  The quantisation decisions are float32, as
the kernel takes them.
"""
import numpy as np

from .formats import E4M3FN_TABLE, bf16_to_f64, round_to_bf16
from .quant import E4M3_MAX, encode_e4m3fn

GROUP = 128


def _bf16_f32(bits) -> np.ndarray:
    return bf16_to_f64(bits).astype(np.float32)


def quant_weight(W_bits, kind: str):
    """bf16 bit patterns W_UK [Lkv, N, P] (kind "uk") or W_UV [Lkv, N, V] (kind "uv") ->
    (codes, w_scale): codes W_K [N, Lkv, P] or W_V [N, V, Lkv] uint8, w_scale float32."""
    W = _bf16_f32(W_bits)
    amax = np.float32(max(float(np.abs(W).max()), 1e-10))
    s = np.float32(round_to_bf16(np.float64(np.float32(E4M3_MAX) / amax)))
    y = round_to_bf16((W * s).astype(np.float64))  # W * s is exact in float32 (8 x 8 bits)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = encode_e4m3fn(y)
    if kind == "uk":
        codes = np.ascontiguousarray(codes.transpose(1, 0, 2))  # [N, Lkv, P]
    elif kind == "uv":
        codes = np.ascontiguousarray(codes.transpose(1, 2, 0))  # [N, V, Lkv]
    else:
        raise ValueError(kind)
    return codes, np.float32(np.float32(1.0) / s)


def quant_act(A_f32):
    """float32 activations [..., K] (K a multiple of 128) -> (codes [..., K] uint8,
    d [..., K / 128] float32 dequantisation scales)."""
    A = np.asarray(A_f32, dtype=np.float32)
    K = A.shape[-1]
    assert K % GROUP == 0
    G = A.reshape(A.shape[:-1] + (K // GROUP, GROUP))
    amax = np.maximum(np.abs(G).max(axis=-1), np.float32(1e-10)).astype(np.float32)
    s = (np.float32(E4M3_MAX) / amax).astype(np.float32)
    y = np.clip((G * s[..., None]).astype(np.float32), np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = encode_e4m3fn(y).reshape(A.shape)
    return codes, (np.float32(1.0) / s).astype(np.float32)


def bmm(A_codes, d, W_codes, w_scale):
    """C[h, m, n] = w_scale * sum_g d[h, m, g] * sum_{k in g} A[h, m, k] W[h, n, k] (float64).
    A_codes [H, M, K], d [H, M, K/128], W_codes [H, Nn, K]."""
    A = E4M3FN_TABLE[A_codes]
    W = E4M3FN_TABLE[W_codes]
    H, M, K = A.shape
    C = np.zeros((H, M, W.shape[1]))
    for g in range(K // GROUP):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        C += d[:, :, g:g + 1].astype(np.float64) * np.matmul(A[:, :, sl], W[:, :, sl].transpose(0, 2, 1))
    return C * np.float64(w_scale)


def absorb_fp8(q_nope_bits, W_K_codes, w_scale):
    """ql_nope [T, N, Lkv] = the fp8 BMM of q_nope [T, N, P] (bf16 bits) with W_K [N, Lkv, P]."""
    q = _bf16_f32(q_nope_bits).transpose(1, 0, 2)  # [N, T, P]
    codes, d = quant_act(q)
    return bmm(codes, d, W_K_codes, w_scale).transpose(1, 0, 2)


def up_fp8(o_latent_bits, W_V_codes, w_scale):
    """o [T, N, V] = the fp8 BMM of o_latent [T, N, Lkv] (bf16 bits) with W_V [N, V, Lkv]."""
    x = _bf16_f32(o_latent_bits).transpose(1, 0, 2)  # [N, T, Lkv]
    codes, d = quant_act(x)
    return bmm(codes, d, W_V_codes, w_scale).transpose(1, 0, 2)
