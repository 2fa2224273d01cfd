// Write of new latent rows into the paged cache (vLLM mla/common.py, MLACommonImpl forward:
// concat_and_cache_mla of k_c_normed and k_pe at slot_mapping, with the fp8 cache quantised
// by the layer's k_scale).
//
// Token i with slot s = slot_mapping[i] >= 0 writes cache row (s / page_size, s % page_size)
// = [kv_c[i, 0:512] | k_pe[i, 0:64]]: copied for a bf16 cache; for an fp8 cache each value
// is x * (1 / k_scale) in fp32 (the reciprocal rounded once), clamped to +-448 and rounded
// to the nearest e4m3fn value, ties to even.  Slots outside [0, num_pages * page_size) are
// skipped (negative slots mark padding tokens).
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

// One thread per 16 bytes of bf16 input: chunk c = 0..71 of token i; chunks 0..63 come
// from kv_c, 64..71 from k_pe (8 values each).  fp8: pairs of chunks make one 16-byte
// output, so a thread takes chunks 2c', 2c'+1 (c' = 0..35).
template <bool FP8>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a) {
  constexpr int PER_TOK = FP8 ? 36 : 72;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.T * PER_TOK) return;
  const int c = (int)(i % PER_TOK);
  const int64_t t = i / PER_TOK;
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= (int64_t)a.num_pages * a.page_size) return;
  const int64_t row = (slot / a.page_size) * a.s_page + (slot % a.page_size) * a.s_tok;  // elements
  auto src8 = [&](int c8) {  // 8 bf16 values of chunk c8 (0..71)
    const uint16_t* p = c8 < 64 ? a.kv_c + t * a.kv_c_s_tok + 8 * c8 : a.k_pe + t * a.k_pe_s_tok + 8 * (c8 - 64);
    return *(const u32x4_t*)p;
  };
  if constexpr (!FP8) {
    *(u32x4_t*)((uint16_t*)a.cache + row + 8 * c) = src8(c);
  } else {
    const u32x4_t v0 = src8(2 * c), v1 = src8(2 * c + 1);
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
    *(u32x4_t*)((uint8_t*)a.cache + row + 16 * c) = out;
  }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, bool fp8, hipStream_t stream) {
  const int64_t n = (int64_t)a.T * (fp8 ? 36 : 72);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (fp8) hipLaunchKernelGGL(cache_write_kernel<true>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(cache_write_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
