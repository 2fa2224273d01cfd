// Static per-tensor fp8 quantisation of the decode query (vLLM mla_attention page,
// MLAAttention forward, decode branch with an fp8 cache: ql_nope and q_pe are
// concatenated and quantised with the layer's static q_scale before the backend call).
//
// q8[t, h, 0:512] = e4m3fn(ql_nope[t, h, :] / q_scale), q8[t, h, 512:576] from q_pe; each
// value is x * (1 / q_scale) in fp32 (the reciprocal rounded once to fp32), clamped to
// +-448 and rounded to the nearest e4m3fn value, ties to even (v_cvt_pk_fp8_f32).
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

// One thread per 16 outputs: chunk c = 0..35 of a (token, head) row; chunks 0..31 come
// from ql_nope, 32..35 from q_pe (32 bytes of bf16 in, 16 bytes of fp8 out).
__global__ __launch_bounds__(256) void concat_quant_q_kernel(QuantArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.T * a.N * 36) return;
  const int c = (int)(i % 36);
  const int64_t r = i / 36;
  const int t = (int)(r / a.N), h = (int)(r % a.N);
  const uint16_t* src = c < 32 ? a.ql + (int64_t)t * a.ql_s_tok + (int64_t)h * a.ql_s_head + 16 * c
                               : a.qpe + (int64_t)t * a.qpe_s_tok + (int64_t)h * a.qpe_s_head + 16 * (c - 32);
  const u32x4_t v0 = *(const u32x4_t*)src, v1 = *(const u32x4_t*)(src + 8);
  float y[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    y[2 * k] = bf16_to_f32((uint16_t)(v0[k] & 0xFFFF));
    y[2 * k + 1] = bf16_to_f32((uint16_t)(v0[k] >> 16));
    y[8 + 2 * k] = bf16_to_f32((uint16_t)(v1[k] & 0xFFFF));
    y[9 + 2 * k] = bf16_to_f32((uint16_t)(v1[k] >> 16));
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) y[k] = fminf(fmaxf(y[k] * a.inv_scale, -448.f), 448.f);
  u32x4_t out;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * k], y[4 * k + 1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * k + 2], y[4 * k + 3], w, true);
    out[k] = (uint32_t)w;
  }
  *(u32x4_t*)(a.q8 + (int64_t)t * a.q8_s_tok + (int64_t)h * a.q8_s_head + 16 * c) = out;
}

}  // namespace

hipError_t launch_concat_quant_q(const QuantArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.T * a.N * 36;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(concat_quant_q_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
