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

// The direct-to-LDS loads set m0 (their LDS base) in the same asm statement and list it
// as clobbered; nothing else in these kernels uses m0.
#pragma clang diagnostic ignored "-Winline-asm"

namespace mla {

namespace {

constexpr int kBN = 128, kBK = 128;

__device__ __forceinline__ int tile_off(int row, int chunk) {  // [row][16 chunks of 16 B]
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}

// One workgroup per (128 n, BM m, head), the tiles of one head on one XCD: with M <= BM
// every weight element is read once (BM = 64 when 128 would leave fewer workgroups than
// compute units; the two m blocks then share the head's weights in that XCD's L2).  K goes in chunks of
// 128; with more than one chunk they go through two register sets: the global loads of
// chunk k+2 are issued once chunk k is in LDS, so they overlap the math of chunk k and the
// staging and math of chunk k+1.
template <bool B_NCONTIG, int BM, bool DB>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int MB = BM / 32;      // 32-row MFMA blocks of the tile's m
  constexpr int AL = BM * 16 / 256;  // A loads per thread and chunk
  __shared__ __attribute__((aligned(16))) char sa[BM * kBK * 2];
  __shared__ __attribute__((aligned(16))) char sb[kBN * kBK * 2];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l32 = l & 31, hh = l >> 5;
  HeadTile ht;
  if (!head_tile((g.Nn + kBN - 1) / kBN, (g.M + BM - 1) / BM, g.H, &ht)) return;
  const int n0 = ht.nb * kBN, m0 = ht.mb * BM, h = ht.h;
  const uint16_t* A = g.A + (int64_t)h * g.a_sh;
  const uint16_t* B = g.B + (int64_t)h * g.b_sh;
  f32x16_t acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

  // global -> registers for one K chunk; two register sets, so the loads of chunk k+2
  // are in flight while chunks k and k+1 are staged and multiplied
  struct Chunk {
    u32x4_t a[AL], b[8];
  };
  auto load = [&](Chunk& r, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {  // A: BM rows x 16 chunks
      const int u = tid + 256 * i, m = u >> 4, c = u & 15;
      r.a[i] = u32x4_t{0, 0, 0, 0};
      if (m0 + m < g.M && k0 + 8 * c < g.K) r.a[i] = *(const u32x4_t*)(A + (int64_t)(m0 + m) * g.a_sm + k0 + 8 * c);
    }
    if constexpr (!B_NCONTIG) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {  // B: 128 rows (n) x 16 chunks (k)
        const int u = tid + 256 * i, n = u >> 4, c = u & 15;
        r.b[i] = u32x4_t{0, 0, 0, 0};
        if (n0 + n < g.Nn && k0 + 8 * c < g.K) r.b[i] = *(const u32x4_t*)(B + (int64_t)(n0 + n) * g.b_sn + k0 + 8 * c);
      }
    } else {  // B: 8 rows (k) x 8 n per thread, transposed on the way to LDS
      const int ko = tid >> 4, no = tid & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = k0 + 8 * ko + e;
        r.b[e] = u32x4_t{0, 0, 0, 0};
        if (k < g.K && n0 + 8 * no < g.Nn) r.b[e] = *(const u32x4_t*)(B + (int64_t)k * g.b_sk + n0 + 8 * no);
      }
    }
  };
  auto store = [&](const Chunk& r) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int u = tid + 256 * i;
      *(u32x4_t*)(sa + tile_off(u >> 4, u & 15)) = r.a[i];
    }
    if constexpr (!B_NCONTIG) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int u = tid + 256 * i;
        *(u32x4_t*)(sb + tile_off(u >> 4, u & 15)) = r.b[i];
      }
    } else {
      const int ko = tid >> 4, no = tid & 15;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4_t o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t x = r.b[2 * k][c >> 1], y = r.b[2 * k + 1][c >> 1];
          o[k] = (c & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
        }
        *(u32x4_t*)(sb + tile_off(8 * no + c, ko)) = o;
      }
    }
  };

  auto chunk = [&](Chunk& r, int k_next) __attribute__((always_inline)) {
    store(r);
    __syncthreads();
    if (k_next < g.K) load(r, k_next);  // in flight during this chunk's and the next one's work
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
  };
  if constexpr (DB) {
    Chunk r0, r1;
    load(r0, 0);
    if (kBK < g.K) load(r1, kBK);
    for (int k0 = 0; k0 < g.K; k0 += 2 * kBK) {
      chunk(r0, k0 + 2 * kBK);
      if (k0 + kBK < g.K) chunk(r1, k0 + 3 * kBK);
    }
  } else {  // one register set (K <= 128: a single chunk), fewer registers per wave
    Chunk r0;
    load(r0, 0);
    for (int k0 = 0; k0 < g.K; k0 += kBK) chunk(r0, k0 + kBK);
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

// ---------------------------------------------------------------------------------
// kv_b_proj of the compute-friendly path (mla/common.py docstring, "Compute Friendly
// Approach"; MLACommonImpl._compute_prefill_context: kv_b_proj of the gathered latent
// rows into k_nope and v): C[s][n] = sum_k A[s][k] * W[k][n] for the two weights W_UK
// and W_UV viewed as [Lkv][N*P] and [Lkv][N*V] (row-major, n contiguous), with all
// S latent rows sharing every weight column.  One launch covers both weights.
//
// Workgroup tile 256 s x 256 n, 4 waves of 128 x 128 (wave w: n half w & 1, s half
// w >> 1), accumulators in AGPRs.  The MFMA computes C^T: A operand = W^T (rows n),
// B operand = A^T (columns s), so a lane ends up with 4 consecutive n of one s.  K goes
// in chunks of 32 through a ring of 4 LDS stages filled by direct-to-LDS loads, three
// chunks ahead.  A stage holds the W chunk as [32 k][256 n] (512-byte rows, 16-byte
// chunk c of row r stored at c ^ 4 (r & 3)) and the A chunk as [256 s][32 k] (64-byte
// rows, chunk c of row r at c ^ ((r >> 2) & 3)).  W^T fragments are read with
// ds_read_b64_tr_b16: in a 16-lane group, lane i reads 4 n at row k0 + (i >> 2),
// column n0 + 4 (i & 3), and receives column n0 + i of rows k0 .. k0 + 3, i.e. 4
// consecutive k of one n.  With these swizzles neither read pattern has bank conflicts.
// Tiles are dealt to XCDs in blocks of 16 n-tiles x all s-tiles, s-major inside a
// block, so the 32 workgroups running on one XCD share 16 n-tiles of weights (4 MB for
// Lkv = 512) in that XCD's L2 and each s-tile of A across 16 workgroups.
constexpr int kKvbStageB = 32768;  // W chunk 16 KB, then A chunk 16 KB
constexpr int kKvbWB = 16384;

__device__ __forceinline__ void kvb_dma(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void kvb_wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__global__ __launch_bounds__(256, 1) void kvb_gemm_kernel(KvbArgs g) {
  __shared__ __attribute__((aligned(1024))) char sm[4 * kKvbStageB];
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  const int bid = blockIdx.x, xcd = bid & 7, jx = bid >> 3;
  if (jx >= g.per_xcd) return;
  const int id = xcd * g.per_xcd + jx;
  if (id >= g.mt * g.nt) return;
  // block of 16 n-tiles x all s-tiles, taken 4 n-tiles at a time, s-major inside: the 32
  // workgroups an XCD runs together cover 8 s-tiles x 4 n-tiles (1 MB of weights)
  const int blk = id / (16 * g.mt), rem = id - blk * 16 * g.mt;
  const int wdt = min(16, g.nt - 16 * blk);
  const int ng = rem / (4 * g.mt), rg = rem - ng * 4 * g.mt;
  const int gw = min(4, wdt - 4 * ng);
  const int s_tile = rg / gw, n_tile = 16 * blk + 4 * ng + rg % gw;
  const int which = n_tile >= g.nt0 ? 1 : 0;
  const uint16_t* W = which ? g.B1 : g.B0;
  uint16_t* C = which ? g.C1 : g.C0;
  const int Nn = which ? g.N1 : g.N0;
  const int s0 = 256 * s_tile, n0 = 256 * (which ? n_tile - g.nt0 : n_tile);

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const uint32_t sm0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)sm;

  // ---- DMA: wave w issues W instructions q = w + 4i (rows 2q, 2q+1) and A instructions
  // q = w + 4i (rows 16q .. 16q+15), i = 0..3; per lane a fixed global offset per
  // instruction (the chunk's k0 added at issue) ----
  const uint16_t* wsrc[4];
  const uint16_t* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = w + 4 * i;
    const int wr = 2 * q + (lane >> 5), wc = (lane & 31) ^ (4 * (wr & 3));
    wsrc[i] = W + (int64_t)wr * Nn + min(n0 + 8 * wc, Nn - 8);
    const int ar = 16 * q + (lane >> 2), ac = (lane & 3) ^ ((lane >> 4) & 3);
    asrc[i] = g.A + (int64_t)min(s0 + ar, g.M - 1) * g.a_s + 8 * ac;
  }
  auto issue = [&](int kc) __attribute__((always_inline)) {
    const uint32_t st = sm0 + (uint32_t)(kc & 3) * kKvbStageB;
    const int64_t k0 = 32 * (int64_t)kc;
#pragma unroll
    for (int i = 0; i < 4; ++i) kvb_dma(wsrc[i] + k0 * Nn, st + 1024 * (w + 4 * i));
#pragma unroll
    for (int i = 0; i < 4; ++i) kvb_dma(asrc[i] + k0, st + kKvbWB + 1024 * (w + 4 * i));
  };

  // ---- fragment addresses within a stage ----
  const int wn = w & 1, ws = w >> 1;
  const int gi = lane & 15, grp = lane >> 4, hh = lane >> 5;
  // W^T (MFMA A operand) for n-block nb, k-step ks, half e4 (0: k 0..3, 1: k 4..7 of the
  // lane half): row 16 ks + 8 hh + 4 e4 + (gi >> 2), n = 128 wn + 32 nb + 16 (grp & 1) + 4 (gi & 3)
  auto wt_addr = [&](int nb, int ks, int e4) __attribute__((always_inline)) {
    const int row = 16 * ks + 8 * hh + 4 * e4 + (gi >> 2);
    const int n = 128 * wn + 32 * nb + 16 * (grp & 1) + 4 * (gi & 3);
    return (uint32_t)(row * 512 + (((n >> 3) ^ (4 * (gi >> 2))) << 4) + 2 * (n & 4));
  };
  // A^T (MFMA B operand) for s-block sb, k-step ks: row 128 ws + 32 sb + lane % 32,
  // chunk 2 ks + hh
  auto at_addr = [&](int sb, int ks) __attribute__((always_inline)) {
    const int row = 128 * ws + 32 * sb + (lane & 31);
    return (uint32_t)(kKvbWB + row * 64 + (((2 * ks + hh) ^ ((row >> 2) & 3)) << 4));
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  auto load_af = [&](u32x4_t (&af)[4], const char* st, int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(const __attribute__((address_space(3))) char*)(st + wt_addr(nb, ks, 0)));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(const __attribute__((address_space(3))) char*)(st + wt_addr(nb, ks, 1)));
      const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
      af[nb] = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
    }
  };
  auto load_bf = [&](u32x4_t (&bf)[4], const char* st, int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) bf[sb] = *(const u32x4_t*)(st + at_addr(sb, ks));
  };
  auto mma = [&](const u32x4_t (&af)[4], const u32x4_t (&bf)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) acc[nb][sb] = mfma32(af[nb], bf[sb], acc[nb][sb]);
  };

  // Chunk kc: k-step 0 runs on fragments loaded during the previous chunk while this
  // chunk's k-step 1 fragments load; then (all waves past the barrier: chunk kc + 1 has
  // landed, the stage of chunk kc - 1 is free) the DMA of chunk kc + 3 goes out and k-step
  // 1 runs while the next chunk's k-step 0 fragments load.
  const int nk = g.K / 32;
  for (int kc = 0; kc < 3 && kc < nk; ++kc) issue(kc);
  if (nk > 2) kvb_wait_vm<16>();
  else if (nk == 2) kvb_wait_vm<8>();
  else kvb_wait_vm<0>();
  __syncthreads();
  u32x4_t af0[4], bf0[4], af1[4], bf1[4];
  load_af(af0, sm, 0);
  load_bf(bf0, sm, 0);
  int kc = 0;
  // steady state, branch-free: every chunk issues the load of chunk kc + 3
  for (; kc + 3 < nk; ++kc) {
    const char* st = sm + (kc & 3) * kKvbStageB;
    load_af(af1, st, 1);
    load_bf(bf1, st, 1);
    mma(af0, bf0);
    kvb_wait_vm<8>();
    __syncthreads();
    issue(kc + 3);
    const char* nx = sm + ((kc + 1) & 3) * kKvbStageB;
    load_af(af0, nx, 0);
    load_bf(bf0, nx, 0);
    mma(af1, bf1);
  }
  // the last (up to) three chunks: nothing more to load
  for (; kc < nk; ++kc) {
    const char* st = sm + (kc & 3) * kKvbStageB;
    load_af(af1, st, 1);
    load_bf(bf1, st, 1);
    mma(af0, bf0);
    if (kc + 1 < nk) {
      // this wave's loads of chunk kc + 1 have landed (8 loads per chunk; chunk kc + 2
      // may still be in flight)
      if (kc + 2 < nk) kvb_wait_vm<8>();
      else kvb_wait_vm<0>();
      __syncthreads();
      if (kc + 3 < nk) issue(kc + 3);
      const char* nx = sm + ((kc + 1) & 3) * kKvbStageB;
      load_af(af0, nx, 0);
      load_bf(bf0, nx, 0);
    }
    mma(af1, bf1);
  }
  __syncthreads();  // every wave is done with the stages: they become the output tile

  // ---- epilogue: wave w's 128 s x 128 n through its 32 KB of LDS ([128 s][16 chunks],
  // chunk c of row r at c ^ (r & 15), its two 8-byte halves swapped in rows with bit 4
  // set, so that the 32 rows one write instruction touches hit distinct banks), then
  // rows of 256 bytes to C ----
  char* ot = sm + w * 32768;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int r = 32 * sb + (lane & 31), n = 32 * nb + 8 * gq + 4 * hh;
        *(u32x2_t*)(ot + r * 256 + (((n >> 3) ^ (r & 15)) << 4) + 8 * (hh ^ ((r >> 4) & 1))) =
            u32x2_t{pack_bf16x2(acc[nb][sb][4 * gq], acc[nb][sb][4 * gq + 1]),
                    pack_bf16x2(acc[nb][sb][4 * gq + 2], acc[nb][sb][4 * gq + 3])};
      }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done (lgkmcnt(0))
  // Non-temporal stores: the output (537 MB for 8192 rows) streams past L2 (measured on the chunked
  // prefill step: 6.90-6.99 -> 6.69-6.74 ms, the GEMM's own time unchanged; the gain is in
  // the attention launches that follow it).
#pragma unroll
  for (int it = 0; it < 32; ++it) {
    const int u = lane + 64 * it, r = u >> 4, c = u & 15;  // (r >> 4) & 1 == (it >> 2) & 1
    const int s = s0 + 128 * ws + r, n = n0 + 128 * wn + 8 * c;
    u32x4_t val = *(const u32x4_t*)(ot + r * 256 + ((c ^ (r & 15)) << 4));
    if ((it >> 2) & 1) val = u32x4_t{val[2], val[3], val[0], val[1]};
    if (s < g.M && n < Nn) __builtin_nontemporal_store(val, (u32x4_t*)(C + (int64_t)s * Nn + n));
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
  if (g.M == 0 || g.H == 0) return hipSuccess;
  const int nb = (g.Nn + kBN - 1) / kBN;
  // 128-row tiles unless that leaves fewer workgroups than the 256 compute units
  const bool big = (int64_t)nb * ((g.M + 127) / 128) * g.H >= 256;
  const dim3 block(256);
  const bool db = g.K > kBK;  // two register sets only where there is a next chunk
  const int64_t tiles = (int64_t)nb * ((g.M + (big ? 127 : 63)) / (big ? 128 : 64)) * g.H;
  const dim3 grid((unsigned)(8 * ((tiles + 7) / 8)));
  if (big) {
    if (g.b_sk == 1) {
      if (db) hipLaunchKernelGGL((gemm_kernel<false, 128, true>), grid, block, 0, stream, g);
      else hipLaunchKernelGGL((gemm_kernel<false, 128, false>), grid, block, 0, stream, g);
    } else {
      if (db) hipLaunchKernelGGL((gemm_kernel<true, 128, true>), grid, block, 0, stream, g);
      else hipLaunchKernelGGL((gemm_kernel<true, 128, false>), grid, block, 0, stream, g);
    }
  } else {
    if (g.b_sk == 1) {
      if (db) hipLaunchKernelGGL((gemm_kernel<false, 64, true>), grid, block, 0, stream, g);
      else hipLaunchKernelGGL((gemm_kernel<false, 64, false>), grid, block, 0, stream, g);
    } else {
      if (db) hipLaunchKernelGGL((gemm_kernel<true, 64, true>), grid, block, 0, stream, g);
      else hipLaunchKernelGGL((gemm_kernel<true, 64, false>), grid, block, 0, stream, g);
    }
  }
  return hipGetLastError();
}

}  // namespace mla

namespace mla {
hipError_t launch_kvb_gemm(KvbArgs g, hipStream_t stream) {
  if (g.M == 0) return hipSuccess;
  g.mt = (g.M + 255) / 256;
  g.nt0 = (g.N0 + 255) / 256;
  g.nt = g.nt0 + (g.N1 + 255) / 256;
  const int64_t tiles = (int64_t)g.mt * g.nt;
  g.per_xcd = (int32_t)((tiles + 7) / 8);
  hipLaunchKernelGGL(kvb_gemm_kernel, dim3((unsigned)(8 * g.per_xcd)), dim3(256), 0, stream, g);
  return hipGetLastError();
}
}  // namespace mla
