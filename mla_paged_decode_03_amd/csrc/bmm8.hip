// fp8 batched GEMMs for the W_UK absorption and the W_UV up-projection (vLLM
// mla/common.py and mla_attention, process_weights_after_loading with the ROCm fp8 BMM:
// per-head weights W_K [N, Lkv, P] and W_V [N, V, Lkv] quantised to e4m3fn with one
// scale per tensor; activations quantised per token in groups of 128 along the
// contracted dimension inside the GEMM).
//
// Weight quantisation (once per weight, one workgroup, no atomics and no scratch): the
// page's bf16 arithmetic, each bf16 operation done in fp32 and rounded to bf16 (ties to
// even): amax = max |W| (at least 1e-10), s = bf16(448 / amax), y = bf16(W * s) clamped
// to +-448, code = e4m3fn(y) (v_cvt_pk_fp8_f32, ties to even); w_scale = fp32(1 / s).
//
// GEMM: C[h][m][n] = w_scale * sum_g d[h][m][g] * sum_{k in g} A8[h][m][k] W8[h][n][k].
// One workgroup (4 waves) per (128 n, BM m, head), the tiles of one head on one XCD (they
// share its weights and activations in that XCD's L2), K in chunks of 128 = one activation
// group, held in registers two chunks ahead when K > 128.  Per chunk: each row's max |a| (the 16
// lanes that hold the row, reduced over their DPP row), then s = 448 / amax and
// d = 1 / s by one thread per row, then the codes of clamp(a * s) into LDS beside the
// copied W rows; each wave runs v_mfma_f32_32x32x64_f8f6f4 over its 32 n rows against
// the BM m columns into a chunk accumulator that is added to the total scaled by that
// row's d (the MFMA computes the tile transposed, so m is the lane column and d a lane
// scalar).
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
constexpr int kRow8 = 144;  // LDS bytes per fp8 row of a K chunk: 128 + 16 pad (36 dwords)

__device__ __forceinline__ float bf16_round(float x) {
  return bf16_to_f32((uint16_t)(pack_bf16x2(x, 0.f) & 0xFFFFu));
}

// 8 fp32 values (already within +-448) -> 8 e4m3fn bytes, ties to even.
__device__ __forceinline__ u32x2_t to_fp8x8(const float* y) {
  u32x2_t out;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * k], y[4 * k + 1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * k + 2], y[4 * k + 3], w, true);
    out[k] = (uint32_t)w;
  }
  return out;
}

__global__ __launch_bounds__(1024) void quant_weight_kernel(const uint16_t* W, int32_t Lkv, int32_t N, int32_t X,
                                                            int32_t which, uint8_t* out, float* w_scale) {
  __shared__ float red[16];
  const int64_t n8 = (int64_t)Lkv * N * X / 8;  // chunks of 8 consecutive elements (X % 8 == 0)
  float mx = 0.f;
  for (int64_t i = threadIdx.x; i < n8; i += 1024) {
    const u32x4_t v = *(const u32x4_t*)(W + 8 * i);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      mx = fmaxf(mx, fmaxf(fabsf(bf16_to_f32((uint16_t)(v[k] & 0xFFFF))), fabsf(bf16_to_f32((uint16_t)(v[k] >> 16)))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, red[i]);
  amax = fmaxf(amax, 1e-10f);
  const float s = bf16_round(448.f / amax);
  for (int64_t i = threadIdx.x; i < n8; i += 1024) {
    // chunk i: W[l][h][x0 .. x0+7]
    const int64_t e = 8 * i;
    const int x0 = (int)(e % X);
    const int64_t lh = e / X;
    const int h = (int)(lh % N), l = (int)(lh / N);
    const u32x4_t v = *(const u32x4_t*)(W + e);
    float y[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      y[2 * k] = bf16_to_f32((uint16_t)(v[k] & 0xFFFF));
      y[2 * k + 1] = bf16_to_f32((uint16_t)(v[k] >> 16));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = fminf(fmaxf(bf16_round(y[k] * s), -448.f), 448.f);
    const u32x2_t q = to_fp8x8(y);
    if (which == 0) {  // W_K[h][l][x] = W_UK[l][h][x]
      *(u32x2_t*)(out + ((int64_t)h * Lkv + l) * X + x0) = q;
    } else {  // W_V[h][x][l] = W_UV[l][h][x]
#pragma unroll
      for (int k = 0; k < 8; ++k) out[((int64_t)h * X + x0 + k) * Lkv + l] = (uint8_t)(q[k >> 2] >> (8 * (k & 3)));
    }
  }
  if (threadIdx.x == 0) *w_scale = 1.f / s;
}

// Maximum of a 32-bit lane value over the 16 lanes of its DPP row (lanes 16r..16r+15):
// quad swaps (xor 1, xor 2), then the half-row and row mirrors pair each quad with the
// others.
__device__ __forceinline__ uint32_t row16_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));  // row_mirror
  return x;
}

template <int BM, bool DB>
__global__ __launch_bounds__(256) void bmm8_kernel(Bmm8Args g) {
  constexpr int MB = BM / 32;
  constexpr int AL = BM * 16 / 256;  // A chunks of 8 bf16 per thread and K chunk
  __shared__ __attribute__((aligned(16))) uint8_t sa[BM * kRow8];
  __shared__ __attribute__((aligned(16))) uint8_t sb[128 * kRow8];
  __shared__ uint32_t ss[BM];  // per row of the chunk: max |a| (bf16 bits), then s (fp32 bits)
  __shared__ float sd[BM];     // per row of the chunk: d = 1 / s
  __shared__ __attribute__((aligned(16))) uint8_t sc[BM * 256];  // bf16 output tile [BM][128]
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l32 = l & 31, hh = l >> 5;
  HeadTile ht;
  if (!head_tile((g.Nn + 127) / 128, (g.M + BM - 1) / BM, g.H, &ht)) return;
  const int n0 = ht.nb * 128, m0 = ht.mb * BM, h = ht.h;
  const uint16_t* A = g.A + (int64_t)h * g.a_sh;
  const uint8_t* B = g.B + (int64_t)h * g.b_sh;
  f32x16_t acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

  // global -> registers for one K chunk; two register sets, so the loads of chunk k+2
  // are in flight while chunks k and k+1 are quantised and multiplied
  struct Chunk {
    u32x4_t a[AL], b[4];
  };
  auto load = [&](Chunk& r, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int u = tid + 256 * i, m = u >> 4, c = u & 15;
      r.a[i] = u32x4_t{0, 0, 0, 0};
      if (m0 + m < g.M) r.a[i] = *(const u32x4_t*)(A + (int64_t)(m0 + m) * g.a_sm + k0 + 8 * c);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i, n = u >> 3, c = u & 7;
      r.b[i] = u32x4_t{0, 0, 0, 0};
      if (n0 + n < g.Nn) r.b[i] = *(const u32x4_t*)(B + (int64_t)(n0 + n) * g.b_sn + k0 + 16 * c);
    }
  };
  // One K chunk = one activation group per row.  Row m of A is held by the 16 lanes
  // u = 16m .. 16m + 15 (one DPP row), 8 values each.
  auto chunk = [&](Chunk& r, int k_next) __attribute__((always_inline)) {
    // the group's max |a| per row: |bf16| compared as 15-bit integers (same order as the
    // values), over the lane's 8 values, then over the row's 16 lanes
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int u = tid + 256 * i, m = u >> 4, c = u & 15;
      uint32_t hi = 0, lo = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hi = max(hi, r.a[i][k] & 0x7FFF0000u);
        lo = max(lo, r.a[i][k] & 0x7FFFu);
      }
      const uint32_t mx = row16_max(max(hi >> 16, lo));
      if (c == 0) ss[m] = mx;
    }
    // W: 128 rows x 8 chunks of 16 bytes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i, n = u >> 3, c = u & 7;
      *(u32x4_t*)(sb + n * kRow8 + 16 * c) = r.b[i];
    }
    __syncthreads();
    // s = 448 / max(amax, 1e-10) and d = 1 / s, both rounded to fp32, once per row
    if (tid < BM) {
      const float s = 448.f / fmaxf(bf16_to_f32((uint16_t)ss[tid]), 1e-10f);
      sd[tid] = 1.f / s;
      ss[tid] = __float_as_uint(s);
    }
    __syncthreads();
    // codes of clamp(a * s, +-448) into the A tile
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int u = tid + 256 * i, m = u >> 4, c = u & 15;
      const float s = __uint_as_float(ss[m]);
      float y[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[2 * k] = fminf(fmaxf(__uint_as_float(r.a[i][k] << 16) * s, -448.f), 448.f);
        y[2 * k + 1] = fminf(fmaxf(__uint_as_float(r.a[i][k] & 0xFFFF0000u) * s, -448.f), 448.f);
      }
      *(u32x2_t*)(sa + m * kRow8 + 8 * c) = to_fp8x8(y);
    }
    __syncthreads();
    if (k_next < g.K) load(r, k_next);
    // operand bytes of lane l: row l % 32, k = 64 ks + 32 (l / 32) .. +31, the same order
    // for both operands (the MFMA pairs equal byte positions of the two lane halves)
    i32x8_t wa[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint8_t* p = sb + (32 * w + l32) * kRow8 + 64 * ks + 32 * hh;
      const u32x4_t lo = *(const u32x4_t*)p, hi = *(const u32x4_t*)(p + 16);
      wa[ks] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x16_t part;
#pragma unroll
      for (int v = 0; v < 16; ++v) part[v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint8_t* p = sa + (32 * mb + l32) * kRow8 + 64 * ks + 32 * hh;
        const u32x4_t lo = *(const u32x4_t*)p, hi = *(const u32x4_t*)(p + 16);
        const i32x8_t xb = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        // e4m3 x e4m3 (format 0 for both), block scales 2^0
        part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa[ks], xb, part, 0, 0, 0, 127, 0, 127);
      }
      const float d = sd[32 * mb + l32];
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][v] += part[v] * d;
    }
    __syncthreads();
  };
  if constexpr (DB) {
    Chunk r0, r1;
    load(r0, 0);
    if (128 < g.K) load(r1, 128);
    for (int k0 = 0; k0 < g.K; k0 += 256) {
      chunk(r0, k0 + 256);
      if (k0 + 128 < g.K) chunk(r1, k0 + 384);
    }
  } else {  // one register set (K = 128: a single chunk), fewer registers per wave
    Chunk r0;
    load(r0, 0);
    for (int k0 = 0; k0 < g.K; k0 += 128) chunk(r0, k0 + 128);
  }
  // Epilogue through LDS: each lane's 4 consecutive n of one m go to the tile as 8 bytes
  // (16-byte chunks of a 256-byte row XOR-swizzled by row), then rows leave as 16-byte
  // pieces, 16 lanes per 256-byte row piece.
  const float ws = *g.w_scale;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int ml = 32 * mb + l32, nl = 32 * w + 8 * gq + 4 * hh;
      *(u32x2_t*)(sc + ml * 256 + (((nl >> 3) ^ (ml & 15)) << 4) + 2 * (nl & 4)) =
          u32x2_t{pack_bf16x2(acc[mb][4 * gq] * ws, acc[mb][4 * gq + 1] * ws),
                  pack_bf16x2(acc[mb][4 * gq + 2] * ws, acc[mb][4 * gq + 3] * ws)};
    }
  __syncthreads();
  uint16_t* C = g.C + (int64_t)h * g.c_sh;
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int u = tid + 256 * i, ml = u >> 4, c = u & 15;
    const int m = m0 + ml, n = n0 + 8 * c;
    if (m < g.M && n < g.Nn)
      *(u32x4_t*)(C + (int64_t)m * g.c_sm + n) = *(const u32x4_t*)(sc + ml * 256 + ((c ^ (ml & 15)) << 4));
  }
}

}  // namespace

hipError_t launch_quant_weight(const uint16_t* W, int32_t Lkv, int32_t N, int32_t X, int32_t which,
                               uint8_t* out, float* w_scale, hipStream_t stream) {
  hipLaunchKernelGGL(quant_weight_kernel, dim3(1), dim3(1024), 0, stream, W, Lkv, N, X, which, out, w_scale);
  return hipGetLastError();
}

hipError_t launch_bmm8(const Bmm8Args& g, hipStream_t stream) {
  if (g.M == 0 || g.H == 0) return hipSuccess;
  const int nb = (g.Nn + 127) / 128;
  // 128-row tiles unless that leaves fewer workgroups than the 256 compute units
  const bool big = (int64_t)nb * ((g.M + 127) / 128) * g.H >= 256;
  const bool db = g.K > 128;  // two register sets only where there is a next chunk
  const int64_t tiles = (int64_t)nb * ((g.M + (big ? 127 : 63)) / (big ? 128 : 64)) * g.H;
  const dim3 grid((unsigned)(8 * ((tiles + 7) / 8)));
  if (big) {
    if (db) hipLaunchKernelGGL((bmm8_kernel<128, true>), grid, dim3(256), 0, stream, g);
    else hipLaunchKernelGGL((bmm8_kernel<128, false>), grid, dim3(256), 0, stream, g);
  } else {
    if (db) hipLaunchKernelGGL((bmm8_kernel<64, true>), grid, dim3(256), 0, stream, g);
    else hipLaunchKernelGGL((bmm8_kernel<64, false>), grid, dim3(256), 0, stream, g);
  }
  return hipGetLastError();
}

}  // namespace mla
