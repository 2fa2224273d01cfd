// Per-head batched bf16 GEMM on MFMA for the W_UK absorption and the W_UV
// up-projection (vLLM mla/common.py module docstring, "Data-Movement Friendly
// Approach": ql_nope = einsum("snh,lnh->snl", q_nope, W_UK) and
// o = einsum("snl,lnv->snv", o_latent, W_UV); the layer runs both as bmm over
// heads).
//
//   C[h][m][n] = sum_k A[h][m][k] * B[h][n][k]
//
// One workgroup (4 waves) computes a 128 or 64 (m) x 128 (n) tile of one head and
// walks K in chunks of 128 staged through LDS.  The MFMA computes the tile
// transposed (rows = n, columns = m) so that each lane ends up with 4
// consecutive n of one m; the output tile goes back through LDS so that rows
// leave as 256-byte pieces (N, P, V and Lkv are multiples of 8).  B is either
// k-contiguous (W_UK: [Lkv][N][P], k = p) or n-contiguous (W_UV: [Lkv][N][V],
// k = l); the latter is transposed 8x8 in registers on its way into LDS.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kBN = 128, kBK = 128;

__device__ __forceinline__ int tile_off(int row, int chunk) {  // [row][16 chunks of 16 B]
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}

// One workgroup per (128 n, BM m, head): with M <= BM every weight element is read once
// (BM = 64 when 128 would leave fewer workgroups than compute units).  K goes in chunks of
// 128; the next chunk's global loads are issued into registers before the current chunk's
// MFMAs, so the loads of chunk k+1 overlap the math of chunk k.
template <bool B_NCONTIG, int BM>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int MB = BM / 32;      // 32-row MFMA blocks of the tile's m
  constexpr int AL = BM * 16 / 256;  // A loads per thread and chunk
  __shared__ __attribute__((aligned(16))) char sa[BM * kBK * 2];
  __shared__ __attribute__((aligned(16))) char sb[kBN * kBK * 2];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l32 = l & 31, hh = l >> 5;
  const int n0 = blockIdx.x * kBN, m0 = blockIdx.y * BM, h = blockIdx.z;
  const uint16_t* A = g.A + (int64_t)h * g.a_sh;
  const uint16_t* B = g.B + (int64_t)h * g.b_sh;
  f32x16_t acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

  // global -> registers for one K chunk
  u32x4_t ra[AL], rb[8];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {  // A: BM rows x 16 chunks
      const int u = tid + 256 * i, m = u >> 4, c = u & 15;
      ra[i] = u32x4_t{0, 0, 0, 0};
      if (m0 + m < g.M && k0 + 8 * c < g.K) ra[i] = *(const u32x4_t*)(A + (int64_t)(m0 + m) * g.a_sm + k0 + 8 * c);
    }
    if constexpr (!B_NCONTIG) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {  // B: 128 rows (n) x 16 chunks (k)
        const int u = tid + 256 * i, n = u >> 4, c = u & 15;
        rb[i] = u32x4_t{0, 0, 0, 0};
        if (n0 + n < g.Nn && k0 + 8 * c < g.K) rb[i] = *(const u32x4_t*)(B + (int64_t)(n0 + n) * g.b_sn + k0 + 8 * c);
      }
    } else {  // B: 8 rows (k) x 8 n per thread, transposed on the way to LDS
      const int ko = tid >> 4, no = tid & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = k0 + 8 * ko + e;
        rb[e] = u32x4_t{0, 0, 0, 0};
        if (k < g.K && n0 + 8 * no < g.Nn) rb[e] = *(const u32x4_t*)(B + (int64_t)k * g.b_sk + n0 + 8 * no);
      }
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int u = tid + 256 * i;
      *(u32x4_t*)(sa + tile_off(u >> 4, u & 15)) = ra[i];
    }
    if constexpr (!B_NCONTIG) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int u = tid + 256 * i;
        *(u32x4_t*)(sb + tile_off(u >> 4, u & 15)) = rb[i];
      }
    } else {
      const int ko = tid >> 4, no = tid & 15;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4_t o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t x = rb[2 * k][c >> 1], y = rb[2 * k + 1][c >> 1];
          o[k] = (c & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
        }
        *(u32x4_t*)(sb + tile_off(8 * no + c, ko)) = o;
      }
    }
  };

  load(0);
  for (int k0 = 0; k0 < g.K; k0 += kBK) {
    store();
    __syncthreads();
    if (k0 + kBK < g.K) load(k0 + kBK);  // in flight during this chunk's MFMAs
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const u32x4_t af = *(const u32x4_t*)(sb + tile_off(32 * w + l32, 2 * ks + hh));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4_t bf = *(const u32x4_t*)(sa + tile_off(32 * mb + l32, 2 * ks + hh));
        acc[mb] = mfma32(af, bf, acc[mb]);
      }
    }
    __syncthreads();
  }
  // Epilogue through LDS (the B tile's space, free after the last barrier): each lane's
  // 4 consecutive n of one m go to the tile as 8 bytes; then rows leave as 16-byte pieces,
  // 16 lanes per 256-byte row piece, instead of 8-byte pieces spread over 32 rows.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int ml = 32 * mb + l32, nl = 32 * w + 8 * gq + 4 * hh;
      *(u32x2_t*)(sb + tile_off(ml, nl >> 3) + 2 * (nl & 4)) =
          u32x2_t{pack_bf16x2(acc[mb][4 * gq], acc[mb][4 * gq + 1]), pack_bf16x2(acc[mb][4 * gq + 2], acc[mb][4 * gq + 3])};
    }
  __syncthreads();
  uint16_t* C = g.C + (int64_t)h * g.c_sh;
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int u = tid + 256 * i, ml = u >> 4, c = u & 15;
    const int m = m0 + ml, n = n0 + 8 * c;
    if (m < g.M && n < g.Nn) *(u32x4_t*)(C + (int64_t)m * g.c_sm + n) = *(const u32x4_t*)(sb + tile_off(ml, c));
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
  if (g.M == 0 || g.H == 0) return hipSuccess;
  const int nb = (g.Nn + kBN - 1) / kBN;
  // 128-row tiles unless that leaves fewer workgroups than the 256 compute units
  const bool big = (int64_t)nb * ((g.M + 127) / 128) * g.H >= 256;
  const dim3 block(256);
  if (big) {
    const dim3 grid(nb, (g.M + 127) / 128, g.H);
    if (g.b_sk == 1) hipLaunchKernelGGL((gemm_kernel<false, 128>), grid, block, 0, stream, g);
    else hipLaunchKernelGGL((gemm_kernel<true, 128>), grid, block, 0, stream, g);
  } else {
    const dim3 grid(nb, (g.M + 63) / 64, g.H);
    if (g.b_sk == 1) hipLaunchKernelGGL((gemm_kernel<false, 64>), grid, block, 0, stream, g);
    else hipLaunchKernelGGL((gemm_kernel<true, 64>), grid, block, 0, stream, g);
  }
  return hipGetLastError();
}

}  // namespace mla
