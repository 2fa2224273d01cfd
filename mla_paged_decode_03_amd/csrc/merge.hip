// LSE merge of partial attention states (split-KV reduce and merge_attn_states).
//
// For states (o_i, lse_i) over disjoint key sets (vLLM mla/common.py module
// docstring, "Chunked Prefill": merge_attn_states of prefix and suffix):
//   m = max lse_i, w_i = exp(lse_i - m), o = sum w_i o_i / sum w_i,
//   lse = m + ln sum w_i;  all -inf -> o = 0, lse = -inf.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

// Split-KV reduce: one workgroup per (request, block of 32 query rows, quarter of the
// 512 columns).  Partial i of a row holds its unnormalised output O_i = sum_j p_j v_j
// times a power-of-two block scale, as fp16, its row sum l_i / kv_scale times the same
// scale, and its lse_i, so o = sum_i exp(lse_i - m) O_i / l_i / z with
// z = sum_i exp(lse_i - m) (the merge above).  The partial outputs of a row block are
// stored in the decode kernels' accumulator order: chunk pair q = 2 (32-column block) + gp
// holds 64 lanes x 8 fp16 values, lane l covering row l % 32 and columns
// 16 gp + 4 (l / 32) .. +3 and 16 gp + 8 + 4 (l / 32) .. +3 of that column block.  Wave w
// of column quarter z merges the 2 chunk pairs of column block 4z + w: one 1 KB load per
// pair and partial, all loads of up to 8 partials (with their LSEs and row sums) issued
// together; the result goes through LDS as a bf16 [32][128] tile and leaves as 256-byte
// row pieces.
constexpr int kTileLd = 128 + 8;  // bf16 row stride of the output tile in LDS
constexpr int kMergeBatch = 8;    // partials whose loads are in flight together
__global__ __launch_bounds__(256) void split_merge_kernel(MergeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[32 * kTileLd];
  const int R = a.Sq * a.N;
  const int red = blockIdx.x, rb = blockIdx.y, zq = blockIdx.z;
  if (red >= a.n_reduce || 32 * rb >= R) return;  // (whole workgroup)
  const int b = a.reduce[3 * red], base = a.reduce[3 * red + 1], n = a.reduce[3 * red + 2];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, rl = l & 31, h2 = l >> 5;
  // this lane's row (rows past R read row R - 1 and are not stored)
  const int r = 32 * rb + rl;
  const float* lse_i = a.ws_lse + (int64_t)base * R + min(r, R - 1);
  const float* l_i = a.ws_l + (int64_t)base * R + min(r, R - 1);
  const int64_t pstride = partial_o_bytes(a.Sq, a.N);
  const int cb = 4 * zq + w;  // column block of this wave
  const char* src = (const char*)a.ws_o + (int64_t)base * pstride + (int64_t)(32 * rb) * kLkv * 2 +
                    16 * (64 * (2 * cb) + l);
  // Every load of the first kMergeBatch partials is issued at once (partial outputs, LSEs
  // and row sums), so the merge waits for one round trip, not one per dependent step.
  u32x4_t x[kMergeBatch][2];
  float lv[kMergeBatch], sv[kMergeBatch];
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k)
    if (k < n) {
      x[k][0] = *(const u32x4_t*)(src + (int64_t)k * pstride);
      x[k][1] = *(const u32x4_t*)(src + (int64_t)k * pstride + 1024);
      sv[k] = lse_i[(int64_t)k * R];
      lv[k] = l_i[(int64_t)k * R];
    }
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k)
    if (k < n) m = fmaxf(m, sv[k]);
  for (int i = kMergeBatch; i < n; ++i) m = fmaxf(m, lse_i[(int64_t)i * R]);
  const bool dead = (m == -INFINITY) || r >= R;
  float z = 0.f;
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k)
    if (k < n) z += fast_exp2((sv[k] - m) * kLog2e);
  for (int i = kMergeBatch; i < n; ++i) z += fast_exp2((lse_i[(int64_t)i * R] - m) * kLog2e);
  const float inv = dead ? 0.f : 1.f / z;
  if (a.lse && zq == 0 && w == 0 && h2 == 0 && r < R) {
    const int t = r / a.N, h = r - t * a.N;
    a.lse[((int64_t)b * a.Sq + t) * a.N + h] = dead ? -INFINITY : m + fast_log2(z) * kLn2;
  }
  // weight exp(lse_i - m) / z over the stored row sum (which carries the value scale and
  // the block scale); rows of a partial that saw no key have lse -inf, weight 0
  float acc[16] = {};  // accumulator element v: column 8 (v / 4) + 4 h2 + v % 4 of the column block
  auto add = [&](const u32x4_t (&xx)[2], float li, float lsev) __attribute__((always_inline)) {
    const float wi = (li > 0.f && !dead) ? fast_exp2((lsev - m) * kLog2e) * inv / li : 0.f;
#pragma unroll
    for (int gp = 0; gp < 2; ++gp)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        acc[8 * gp + 2 * d] += wi * f16_lo(xx[gp][d]);
        acc[8 * gp + 2 * d + 1] += wi * f16_hi(xx[gp][d]);
      }
  };
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k)
    if (k < n) add(x[k], lv[k], sv[k]);
  for (int i = kMergeBatch; i < n; ++i) {
    const u32x4_t xx[2] = {*(const u32x4_t*)(src + (int64_t)i * pstride),
                           *(const u32x4_t*)(src + (int64_t)i * pstride + 1024)};
    add(xx, l_i[(int64_t)i * R], lse_i[(int64_t)i * R]);
  }
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    const int col = 32 * w + 8 * gq + 4 * h2;  // within this quarter
    *(u32x2_t*)(tile + rl * kTileLd + col) = u32x2_t{pack_bf16x2(acc[4 * gq], acc[4 * gq + 1]),
                                                     pack_bf16x2(acc[4 * gq + 2], acc[4 * gq + 3])};
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + 256 * k, row = idx >> 4, c8 = idx & 15;
    const int rr = 32 * rb + row;
    if (rr >= R) continue;
    const int t = rr / a.N, h = rr - t * a.N;
    uint16_t* dst = a.o + ((int64_t)b * a.Sq + t) * a.o_s_tok + (int64_t)h * a.o_s_head + 128 * zq + 8 * c8;
    *(u32x4_t*)dst = *(const u32x4_t*)(tile + row * kTileLd + 8 * c8);
  }
}

__device__ __forceinline__ void load8(const void* p, bool fp32, float* x) {
  if (fp32) {
    const f32x4_t a = *(const f32x4_t*)p;
    const f32x4_t b = *((const f32x4_t*)p + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[4 + e] = b[e];
    }
  } else {
    const u32x4_t v = *(const u32x4_t*)p;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_to_f32((uint16_t)(v[k] & 0xFFFF));
      x[2 * k + 1] = bf16_to_f32((uint16_t)(v[k] >> 16));
    }
  }
}

// One row per lpr lanes (lpr a power of two covering D / 8 chunks of 8 values, at most 64),
// so a wave merges 64 / lpr rows at once when D is small.
__global__ __launch_bounds__(256) void merge_two_kernel(void* out, float* out_lse, const void* po,
                                                        const float* plse, const void* so,
                                                        const float* slse, int64_t rows, int D,
                                                        int fp32, int lpr) {
  const int rpw = 64 / lpr;  // rows per wave
  const int w = threadIdx.x >> 6, lw = threadIdx.x & 63, l = lw & (lpr - 1);
  const int64_t r = ((int64_t)blockIdx.x * 4 + w) * rpw + lw / lpr;
  if (r >= rows) return;
  const float lp = plse[r], ls = slse[r];
  const float m = fmaxf(lp, ls);
  float wp = 0.f, wsf = 0.f, lse = -INFINITY;
  if (m != -INFINITY) {
    wp = fast_exp2((lp - m) * kLog2e);
    wsf = fast_exp2((ls - m) * kLog2e);
    const float z = wp + wsf;
    lse = m + fast_log2(z) * kLn2;
    wp /= z;
    wsf /= z;
  }
  const int esz = fp32 ? 4 : 2;
  for (int c = 8 * l; c < D; c += 8 * lpr) {
    float x[8], y[8];
    const int64_t off = (r * D + c) * esz;
    load8((const char*)po + off, fp32, x);
    load8((const char*)so + off, fp32, y);
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = wp * x[e] + wsf * y[e];
    if (fp32) {
      *(f32x4_t*)((char*)out + off) = f32x4_t{o[0], o[1], o[2], o[3]};
      *((f32x4_t*)((char*)out + off) + 1) = f32x4_t{o[4], o[5], o[6], o[7]};
    } else {
      *(u32x4_t*)((char*)out + off) = u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                              pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
    }
  }
  if (out_lse && l == 0) out_lse[r] = lse;
}

__global__ void gather_rows_kernel(const int32_t* bt, int64_t bt_s, const int32_t* seq_lens,
                                   const int64_t* offsets, int page_size, int64_t* rows) {
  const int b = blockIdx.x;
  const int L = seq_lens[b];
  const int32_t* row = bt + (int64_t)b * bt_s;
  for (int j = threadIdx.x; j < L; j += blockDim.x)
    rows[offsets[b] + j] = (int64_t)row[j / page_size] * page_size + j % page_size;
}

}  // namespace

hipError_t launch_split_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.n_reduce == 0) return hipSuccess;
  const int R = a.Sq * a.N;
  const dim3 grid(a.n_reduce, (R + 31) / 32, 4), block(256);
  hipLaunchKernelGGL(split_merge_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge_two(void* out, float* out_lse, const void* prefix_o, const float* prefix_lse,
                            const void* suffix_o, const float* suffix_lse, int64_t rows, int32_t D,
                            bool fp32, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  int lpr = 1;
  while (lpr < 64 && 8 * lpr < D) lpr *= 2;
  const int64_t rows_per_wg = 4 * (64 / lpr);
  const dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg)), block(256);
  hipLaunchKernelGGL(merge_two_kernel, grid, block, 0, stream, out, out_lse, prefix_o, prefix_lse,
                     suffix_o, suffix_lse, rows, D, (int)fp32, lpr);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const int32_t* block_table, int64_t bt_s, const int32_t* seq_lens,
                              const int64_t* offsets, int32_t B, int32_t page_size, int64_t* rows,
                              hipStream_t stream) {
  hipLaunchKernelGGL(gather_rows_kernel, dim3(B), dim3(256), 0, stream, block_table, bt_s, seq_lens,
                     offsets, page_size, rows);
  return hipGetLastError();
}

}  // namespace mla
