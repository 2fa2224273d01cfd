// Chunked prefill, compute-friendly form, for gfx950 (vLLM mla/common.py module
// docstring, "Chunked Prefill"; MLACommonImpl._compute_prefill_context / forward_mha).
//
// Keys and values are up-projected per head (k_nope = kv_c W_UK, v = kv_c W_UV, done by
// the GEMM of gemm.hip), the rope part k_pe is shared by every head, and each head runs
// plain multi-head attention with QK width P+R = 192 and value width V = 128.  The
// context is visited in chunks: the chunk's latent rows are gathered from the paged
// cache (and dequantised) into a contiguous workspace, up-projected, attended to without
// a mask, and the chunk outputs are merged by LSE; the new tokens attend to themselves
// causally, and one last merge combines the two.
//
// Attention (prefill_attn_pipe_kernel, for both the causal and the unmasked launches).
// Per tile of 32 keys:
//   S^T[key][query] = K[key][:] . Q[query][:]     (12 MFMAs 32x32x16 per 32 queries)
//   online softmax per query (the 16 logits of a lane plus its partner lane l^32)
//   O^T[v][query]  += V^T[v][key] . P^T[key][query] (8 MFMAs)
// so every per-query quantity (maximum, row sum, rescale factor) is a per-lane scalar.
// V is read as V^T from row-major LDS rows by transposing reads, and the QK takes the K
// rows in a permuted key order so that P^T needs no shuffle.  One workgroup per CU,
// blocks of 256 queries, each wave two sub-blocks of 32, K/V by direct-to-LDS loads into
// a 4-stage ring, and the QK of the next tile interleaved with the softmax (described
// with the kernel below).  Causal launches give each workgroup a pair of query blocks
// whose causal key ranges add up to the same length.  Work items of one head are dealt
// to one XCD, so that they share its L2 for the head's K/V.
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

// The direct-to-LDS loads set m0 (their LDS base) in the same asm statement and list it
// as clobbered; nothing else in these kernels uses m0.
#pragma clang diagnostic ignored "-Winline-asm"

namespace mla {

namespace {

constexpr int kPT = 32;          // keys per tile
constexpr int kPN = 128;         // P (k_nope / q_nope width)
constexpr int kPR = 64;          // R (rope width)
constexpr int kPV = 128;         // V (value width)

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// S^T row i of the QK MFMA holds tile key pi(i): then the 8 keys of P.V k-step s in lane
// half h are {16s + h + 4e} and {16s + 2 + h + 4e} (e = 0..3), the 4-key strides that
// one transposing LDS read delivers.
__device__ __forceinline__ int pi_key(int i) { return ((i >> 2) & 3) + 4 * (i & 3) + 16 * (i >> 4); }

// 8 bf16 of V^T (this lane's value column, 8 keys) from the row-major V tile: two
// ds_read_b64_tr_b16 (16-lane group: lane j addresses row x + 4(j / 4), columns
// 4(j % 4) .. +3 and receives column j of rows x, x+4, x+8, x+12).
__device__ __forceinline__ u32x4_t read_vt(const uint16_t* p0, const uint16_t* p1) {
  const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const lds_char*)(const void*)p0);
  const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const lds_char*)(const void*)p1);
  const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0), w1 = __builtin_bit_cast(u32x2_t, v1);
  return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
}

constexpr float kRescaleAt = 8.f;  // log2 units a tile maximum may exceed the reference by

// ---------------------------------------------------------------------------------
// Pipelined attention kernel: one workgroup (4 waves, one per SIMD) per (request, head,
// block of 256 queries); wave w owns queries 64w .. 64w+63 as two sub-blocks of 32 (one
// per lane column of the MFMA), so every K or V fragment read from LDS feeds two MFMAs.
// K and V tiles (32 keys) go HBM/L2 -> LDS by direct-to-LDS loads into a ring of 4
// stages, two tiles ahead, with one barrier per tile.  A stage holds K_nope [32][128],
// K_pe [32][64] and V [32][128] as unpadded rows whose 16-byte chunks are XOR-swizzled
// by key (the DMA writes each lane's 16 bytes in lane order, so the swizzle is applied
// on the global side): chunk c of key k sits in slot c ^ (k % 16) of a K_nope row,
// c ^ ((k / 2) % 8) of a K_pe row and c ^ 4 ((k / 4) % 4) of a V row, which puts the 16
// keys of one b128 K read, and the 4 rows x 2 chunks of one transposing V read, on
// distinct banks.  Each tile is 20 DMA instructions of 64 lanes, 5 per wave at fixed
// places (K_nope keys 4j..4j+3 for j = w, w + 4; K_pe keys 8w..8w+7; V like K_nope).
// The reference maximum moves lazily (kRescaleAt), so O is rescaled only when a logit
// exceeds it by 2^8.
constexpr int kQB = 256;               // queries per workgroup
constexpr int kKnB = kPT * kPN * 2;    // 8192 bytes
constexpr int kKpB = kPT * kPR * 2;    // 4096
constexpr int kVB = kPT * kPV * 2;     // 8192
constexpr int kStg = kKnB + kKpB + kVB;  // 20480
constexpr int kNStg = 4;
constexpr int kDmaPerWave = 5;

__device__ __forceinline__ void pdma16(const void* gbase, uint32_t voff, uint32_t lds_base) {
  // uniform: the tile's base in SGPRs (readfirstlane returns int: each half is taken as
  // unsigned, or a low word >= 2^31 would sign-extend into the high one)
  const uint64_t g = (uint64_t)(uintptr_t)gbase;
  const uint64_t gs = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)g) |
                      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(g >> 32)) << 32);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"((const void*)gs),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
// P.V MFMA with its accumulator pinned to AGPRs (inline asm: the compiler then leaves the
// AGPRs to O and never moves it through VGPRs).  The compiler does not model the hazards
// of inline MFMAs: each carries the 3 wait states that a VALU write of its operands just
// before needs; a VALU read of O follows the last one only after the next tile's QK, or
// behind pv_drain.
__device__ __forceinline__ void pv_mfma(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// QK MFMAs: S^T accumulates in VGPRs (read by the softmax one step later, after the
// P.V MFMAs, so with no wait states of their own), the query operand comes from AGPRs.
__device__ __forceinline__ void qk_first(f32x16_t& d, const u32x4_t& k, const u32x4_t& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "a"(q));
}
__device__ __forceinline__ void qk_acc(f32x16_t& d, const u32x4_t& k, const u32x4_t& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
}
// The same with the 3 wait states that a VALU write of an operand just before needs (the
// first tile's QK, before the loop: the compiler may move the queries between registers).
__device__ __forceinline__ void qk_first_s(f32x16_t& d, const u32x4_t& k, const u32x4_t& q) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "a"(q));
}
__device__ __forceinline__ void qk_acc_s(f32x16_t& d, const u32x4_t& k, const u32x4_t& q) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
}
// Maxima as plain instructions: fmaxf would first canonicalise every operand that
// comes out of inline asm (one more VALU op each); the logits are never NaN.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
__device__ __forceinline__ float vmax2(float a, float b) {
  float d;
  asm("v_max_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}
// Maximum over the lane pair (l, l ^ 32), in one statement: after the swap of the copy's
// low half with x's high half, lane l holds x of lanes l % 32 and l % 32 + 32.
__device__ __forceinline__ float pair_max(float x) {
  float t;
  asm volatile("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_max_f32 %0, %0, %1"
               : "+v"(x), "=&v"(t));
  return x;
}
// Calls f(std::integral_constant<int, K>) for K = 0..N-1 in order, as straight-line code.
template <int N, typename F>
__device__ __forceinline__ void pstatic_for(F&& f) {
  [&]<int... K>(std::integer_sequence<int, K...>) {
    (f(std::integral_constant<int, K>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}
// The same without leading wait states, for operands that no VALU op wrote just before
// (V^T from LDS, P from the softmax's earlier slots).
__device__ __forceinline__ void pv_mfma_nw(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// O in AGPRs up to this point: the compiler copies one block to VGPRs where it is read,
// not all of O at once.
__device__ __forceinline__ void pv_fence(f32x16_t& d) { asm volatile("" : "+a"(d)::"memory"); }
// The 3 wait states between VALU writes of O (rescale) and the MFMAs that read it, with O
// in AGPRs at this point.
__device__ __forceinline__ void pv_written(f32x16_t (&o)[4]) {
  asm volatile("s_nop 2" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
}
// 16 wait states after the last P.V MFMA, before VALU reads of O.
__device__ __forceinline__ void pv_drain(f32x16_t (&o)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 1" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
}
template <int N>
__device__ __forceinline__ void pwait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void pbarrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // s_waitcnt lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}
// byte offset, from the tile's first key, of the global chunk that DMA lane `lane` of
// region instruction j moves (keys clamped to `kmax`, the tile's last key that exists)
template <int REG>  // 0: K_nope, 1: K_pe, 2: V
__device__ __forceinline__ uint32_t pdma_off(int j, int lane, int kmax, int64_t stok) {
  const int key = REG == 1 ? 8 * j + (lane >> 3) : 4 * j + (lane >> 4);
  const int slot = REG == 1 ? (lane & 7) : (lane & 15);
  const int col = REG == 0 ? slot ^ (key & 15) : (REG == 1 ? slot ^ ((key >> 1) & 7) : slot ^ (4 * ((key >> 2) & 3)));
  return (uint32_t)(2 * stok * min(key, kmax) + 16 * col);
}

__global__ __launch_bounds__(256, 1) void prefill_attn_pipe_kernel(PrefillAttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char sm[kNStg * kStg];
  const int L = blockIdx.x;
  const int item = (L & 7) * a.per_xcd + (L >> 3);
  if (item >= a.items) return;  // (whole workgroup)
  // An item is one query block, or with causal masks a pair of blocks (nqb - 1 - p, p)
  // whose key ranges add up to nqb + 1 blocks' worth, so that every pair costs the same.
  const int nqb = a.q_blocks;
  const int nit = a.causal ? (nqb + 1) / 2 : nqb;  // items per (request, head)
  const int pr = item % nit;
  const int h = (item / nit) % a.N, b = item / nit / a.N;
  const int q0 = a.cu_q[b], Sq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], Sk = a.cu_k[b + 1] - k0;
#pragma unroll 1
  for (int pass = 0; pass < (a.causal && 2 * pr + 1 < nqb ? 2 : 1); ++pass) {
  const int qb = pass == 0 ? nqb - 1 - pr : pr;
  if (kQB * qb >= Sq) continue;  // (whole workgroup)
  if (pass == 1) __syncthreads();  // the first block's epilogue staged through the stages
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qlast = min(Sq, kQB * qb + kQB) - 1;
  const int nkeys = a.causal ? max(0, min(Sk, qlast + Sk - Sq + 1)) : Sk;
  const int ntiles = (nkeys + kPT - 1) / kPT;
  // tiles below this key count need no mask for any query of the workgroup
  const int unmasked = a.causal ? max(0, min(Sk, kQB * qb + Sk - Sq + 1)) : Sk;
  const uint32_t sm0 = (uint32_t)(uintptr_t)(const lds_char*)sm;
  const int64_t kn_st = a.kn_s_tok, kp_st = a.kp_s_tok, v_st = a.v_s_tok;
  const uint16_t* kn_b = a.k_nope + (int64_t)k0 * kn_st + (int64_t)h * a.kn_s_head;
  const uint16_t* kp_b = a.k_pe + (int64_t)k0 * kp_st;
  const uint16_t* v_b = a.v + (int64_t)k0 * v_st + (int64_t)h * a.v_s_head;

  // ---- DMA of tile kt into stage kt % 4 ----
  uint32_t dof[kDmaPerWave];
  dof[0] = pdma_off<0>(w, lane, kPT - 1, kn_st);
  dof[1] = pdma_off<0>(w + 4, lane, kPT - 1, kn_st);
  dof[2] = pdma_off<1>(w, lane, kPT - 1, kp_st);
  dof[3] = pdma_off<2>(w, lane, kPT - 1, v_st);
  dof[4] = pdma_off<2>(w + 4, lane, kPT - 1, v_st);
  auto issue = [&](int kt) __attribute__((always_inline)) {
    const uint32_t st = sm0 + (uint32_t)(kt % kNStg) * kStg;
    const int kmax = min(kPT, Sk - kPT * kt) - 1;
    uint32_t o0 = dof[0], o1 = dof[1], o2 = dof[2], o3 = dof[3], o4 = dof[4];
    if (kmax < kPT - 1) {  // (uniform) the request's keys end inside this tile: clamp
      o0 = pdma_off<0>(w, lane, kmax, kn_st);
      o1 = pdma_off<0>(w + 4, lane, kmax, kn_st);
      o2 = pdma_off<1>(w, lane, kmax, kp_st);
      o3 = pdma_off<2>(w, lane, kmax, v_st);
      o4 = pdma_off<2>(w + 4, lane, kmax, v_st);
    }
    const int64_t kk = (int64_t)kPT * kt;
    pdma16(kn_b + kk * kn_st, o0, st + 1024 * w);
    pdma16(kn_b + kk * kn_st, o1, st + 1024 * (w + 4));
    pdma16(kp_b + kk * kp_st, o2, st + kKnB + 1024 * w);
    pdma16(v_b + kk * v_st, o3, st + kKnB + kKpB + 1024 * w);
    pdma16(v_b + kk * v_st, o4, st + kKnB + kKpB + 1024 * (w + 4));
  };
  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  // ---- queries of both sub-blocks, loaded after the DMA of tiles 0 and 1 (the
  // compiler's wait for them, which counts only its own loads, then also covers those
  // older DMA loads; the latencies overlap): sub-block j, k-step ks covers dims
  // 16 ks + 8 hh .. +7 (q_nope for ks < 8, q_pe after); rows past Sq load the block's
  // last query and are never stored ----
  u32x4_t qf[2][12];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qi = min(kQB * qb + 64 * w + 32 * j + l32, Sq - 1);
    const int64_t t = (int64_t)q0 + qi;
    const uint16_t* qn = a.q_nope + t * a.qn_s_tok + (int64_t)h * a.qn_s_head + 8 * hh;
    const uint16_t* qp = a.q_pe + t * a.qp_s_tok + (int64_t)h * a.qp_s_head + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks)
      qf[j][ks] = ks < 8 ? *(const u32x4_t*)(qn + 16 * ks) : *(const u32x4_t*)(qp + 16 * (ks - 8));
  }

  // the compiler waits for the queries here (and with them for tiles 0 and 1), not
  // inside the loop, where its wait would also drain the DMA loads in flight
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) asm volatile("" : "+a"(qf[j][ks]));  // (kept in AGPRs)
  if (ntiles > 2) issue(2);

  f32x16_t o[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[j][vb][e] = 0.f;
  // (an accumulator operand in AGPRs: the compiler then keeps every MFMA result there)
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int vb = 0; vb < 4; ++vb) asm volatile("" : "+a"(o[j][vb]));
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  const float cs = a.scale_log2;
  // K fragment reads: row krow (permuted key order), chunk 2 ks + hh, swizzled
  const int krow = pi_key(l32);
  const int kn_row = krow * (2 * kPN), kp_row = kKnB + krow * (2 * kPR);
  const int kn_x = krow & 15, kp_x = (krow >> 1) & 7;
  // transposing V reads: lane row hh + 4 q (q = (l % 16) / 4), chunk 2 ((l / 16) % 2) +
  // (l % 4) / 2 of value block vb, byte 8 (l % 2); swizzle 4 q, so the block index vb
  // meets it as vb ^ q; k-step s adds 16 rows, the second read 2 rows
  const int vq = (lane & 15) >> 2;
  const int vbase = kKnB + kKpB + (hh + 4 * vq) * (2 * kPV) + 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) +
                    8 * (lane & 1);
  int qlim[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qi = kQB * qb + 64 * w + 32 * j + l32;
    qlim[j] = a.causal ? qi + Sk - Sq : Sk - 1;  // last key this lane's query sees
  }

  // K fragment ks of tile kt (row krow, chunk 2 ks + hh, swizzled)
  auto kread = [&](int kt, int ks) __attribute__((always_inline)) {
    const char* st = sm + (kt % kNStg) * kStg;
    return ks < 8 ? *(const u32x4_t*)(st + kn_row + 16 * ((2 * ks + hh) ^ kn_x))
                  : *(const u32x4_t*)(st + kp_row + 16 * ((2 * (ks - 8) + hh) ^ kp_x));
  };
  // lane holds S^T rows 8 gq + 4 hh + e (index 4 gq + e): tile keys pi of those
  auto mask = [&](int kt, f32x16_t (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const int key = kt * kPT + pi_key(8 * (idx >> 2) + 4 * hh + (idx & 3));
        if (key > qlim[j] || key >= Sk) s[j][idx] = -INFINITY;
      }
  };
  // Online softmax of one tile for both sub-blocks, without branches, cut into 26 micro
  // steps (13 per sub-block) that the QK MFMAs of the next tile interleave: the tile
  // maximum, the moved reference (lazily, by kRescaleAt) with the factor alpha for O and l,
  // then per pair of logits p = 2^(s cs - m), the row sum and P^T as bf16.
  struct Soft {
    float mx[2], mu[2], ls[2], alpha[2];
    u32x4_t pb[2][2];
  };
  auto micro = [&](auto kc, f32x16_t (&s)[2], Soft& z) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value, j = k / 13, r = k % 13;
    if constexpr (r == 0) {
      z.mx[j] = vmax3(vmax3(s[j][0], s[j][1], s[j][2]), s[j][3], s[j][4]);
    } else if constexpr (r < 3) {
      z.mx[j] = vmax3(vmax3(z.mx[j], s[j][4 * r + 1], s[j][4 * r + 2]), s[j][4 * r + 3], s[j][4 * r + 4]);
    } else if constexpr (r == 3) {
      z.mx[j] = pair_max(vmax2(vmax3(z.mx[j], s[j][13], s[j][14]), s[j][15])) * cs;
    } else if constexpr (r == 4) {
      const float m_new = z.mx[j] > m[j] + kRescaleAt ? z.mx[j] : m[j];
      z.alpha[j] = m_new == m[j] ? 1.f : fast_exp2(m[j] - m_new);  // 0 while m is -inf
      m[j] = m_new;
      z.mu[j] = m_new == -INFINITY ? 0.f : m_new;
      z.ls[j] = lsum[j] * z.alpha[j];
    } else {
      constexpr int e = r - 5;  // logits 2e, 2e + 1
      const float xa = fast_exp2(fmaf(s[j][2 * e], cs, -z.mu[j]));
      const float xb = fast_exp2(fmaf(s[j][2 * e + 1], cs, -z.mu[j]));
      z.ls[j] += xa;
      z.ls[j] += xb;
      z.pb[j][e >> 2][e & 3] = pack_bf16x2(xa, xb);
      if constexpr (e == 7) lsum[j] = z.ls[j];
    }
  };
  // O held P.V up to the previous tile against the old reference (rare)
  auto rescale = [&](const float (&alpha)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (__any(alpha[j] != 1.f)) {
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) {
          pv_fence(o[j][vb]);
#pragma unroll
          for (int e = 0; e < 16; ++e) o[j][vb][e] *= alpha[j];
        }
        pv_written(o[j]);
      }
  };
  // V^T fragment i (value block i / 2, k-step i % 2) of tile kt: two transposing reads
  auto vread = [&](int kt, int i) __attribute__((always_inline)) {
    const char* st = sm + (kt % kNStg) * kStg;
    const uint16_t* p = (const uint16_t*)(st + vbase + 64 * ((i >> 1) ^ vq));
    return read_vt(p + 16 * (i & 1) * kPV, p + (16 * (i & 1) + 2) * kPV);
  };
  // Software pipeline over tiles: step t runs the QK of tile t + 1 on the MFMA unit while
  // the VALU computes the softmax of tile t (one slot of micro steps after each MFMA; the
  // scheduling barriers keep every slot in place), then the P.V of tile t.  The barrier of
  // step t publishes tile t + 1 and frees the stage of tile t - 1 for the DMA of tile t + 3.
  f32x16_t sA[2], sB[2];
  if (ntiles > 0) {
    pbarrier();  // tile 0 (each wave waited for its own part with the queries)
    u32x4_t kf[12];
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) kf[ks] = kread(0, ks);
#pragma unroll
    for (int ks = 0; ks < 12; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (ks == 0) qk_first_s(sA[j], kf[0], qf[j][0]);
        else qk_acc_s(sA[j], kf[ks], qf[j][ks]);
      }
    // the softmax reads S next: the wait states after the last MFMA
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 1" : "+v"(sA[0]), "+v"(sA[1]));
  }
  auto step = [&](int t, f32x16_t (&sc)[2], f32x16_t (&sn)[2]) __attribute__((always_inline)) {
    if (t + 2 < ntiles) pwait_vm<kDmaPerWave>();
    else pwait_vm<0>();
    pbarrier();
    if (t + 3 < ntiles) issue(t + 3);
    if (t * kPT + kPT > unmasked) mask(t, sc);  // (uniform) on the diagonal or past Sk
    Soft z;
    u32x4_t vf[8];
    // phase 1: the QK of tile t + 1 with the softmax of sub-block 0 and the reference of
    // sub-block 1 (micro steps 0..17), the V^T reads of tile t in the last 8 slots
    {
      u32x4_t kf[12];  // read two fragments ahead of their MFMAs
      kf[0] = kread(t + 1, 0);
      kf[1] = kread(t + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      pstatic_for<24>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value, ks = i >> 1, j = i & 1;
        if constexpr (j == 0 && ks + 2 < 12) kf[ks + 2] = kread(t + 1, ks + 2);
        if constexpr (i >= 16) vf[i - 16] = vread(t, i - 16);
        if constexpr (ks == 0) qk_first(sn[j], kf[0], qf[j][0]);
        else qk_acc(sn[j], kf[ks], qf[j][ks]);
        constexpr int lo = i * 18 / 24, hi = (i + 1) * 18 / 24;
        pstatic_for<hi - lo>([&](auto kc) __attribute__((always_inline)) {
          micro(std::integral_constant<int, lo + decltype(kc)::value>{}, sc, z);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    // P of sub-block 0 and both factors are complete here (not sunk past the branch)
    asm volatile("" ::"v"(z.pb[0][0]), "v"(z.pb[0][1]), "v"(lsum[0]), "v"(z.mu[1]), "v"(z.ls[1]));
    rescale(z.alpha);
    // phase 2: P.V of sub-block 0 with the exponentials of sub-block 1 (micro steps
    // 18..25), then P.V of sub-block 1 (k-step outer: dependent MFMAs are 4 apart)
    __builtin_amdgcn_sched_barrier(0);
    pstatic_for<8>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, ss = i >> 2, vb = i & 3;
      pv_mfma_nw(o[0][vb], vf[2 * vb + ss], z.pb[0][ss]);
      micro(std::integral_constant<int, 18 + i>{}, sc, z);
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        if (ss == 0 && vb == 0) pv_mfma(o[1][vb], vf[2 * vb + ss], z.pb[1][ss]);  // P just written
        else pv_mfma_nw(o[1][vb], vf[2 * vb + ss], z.pb[1][ss]);
      }
  };
  // Every step is the steady-state one: the last tile's step also runs a QK, of a tile
  // that does not exist (stale LDS into S registers nobody reads; 24 MFMAs per workgroup),
  // so the loop is the only copy of the step and needs no separately scheduled tail.
  for (int t = 0; t < ntiles; t += 2) {
    step(t, sA, sB);
    if (t + 1 < ntiles) step(t + 1, sB, sA);
  }
  pv_drain(o[0]);  // the wait states before anything reads or moves O
  pv_drain(o[1]);

  // ---- epilogue per sub-block: o = O / l (bf16), lse = ln sum exp; with a running state
  // (prev_o, prev_lse) its LSE merge with this result.  O / l goes through LDS as fp32, 64
  // columns at a time, so that each store writes whole 128-byte rows of o (8 lanes a row)
  // rather than 16 bytes into each of 32 rows (partial lines, written back about three
  // times over).  Wave w uses an 8.5 KB region of stage (ntiles + w / 2) % 4: no DMA is in
  // flight any more, and every wave has passed the barrier after which that stage (tile
  // ntiles - 4 or ntiles - 3, or one never filled) is read by nobody but the unused QK of
  // the last step.
  constexpr int kEpRow = 68;  // floats per staged row (64 + 4 pad: b128 accesses free of conflicts)
  float* ep = (float*)(sm + ((ntiles + (w >> 1)) % kNStg) * kStg) + (w & 1) * (32 * kEpRow);
  float* epf = (float*)(sm + ((ntiles + (w >> 1)) % kNStg) * kStg) + 2 * 32 * kEpRow + (w & 1) * 32;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float lrow = half_sum(lsum[j]);
    const int qi = kQB * qb + 64 * w + 32 * j + l32;
    const int64_t t = (int64_t)q0 + min(qi, Sq - 1);
    const float lse_new = lrow > 0.f ? (m[j] + fast_log2(lrow)) * kLn2 : -INFINITY;
    float f_new = lrow > 0.f ? 1.f / lrow : 0.f, f_prev = 0.f, lse_out = lse_new;
    if (a.prev_o && qi < Sq) {
      const float lp = a.prev_lse[t * a.N + h];
      const float mm = fmaxf(lp, lse_new);
      if (mm == -INFINITY) {
        f_new = 0.f;
      } else {
        const float wp = fast_exp2((lp - mm) * kLog2e), wn = fast_exp2((lse_new - mm) * kLog2e);
        const float z = wp + wn;
        f_prev = wp / z;
        f_new *= wn / z;
        lse_out = mm + fast_log2(z) * kLn2;
      }
    }
    if (a.lse && hh == 0 && qi < Sq) a.lse[t * a.N + h] = lse_out;
    if (hh == 0) epf[l32] = f_prev;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // this lane's part of rows l32: columns 32 c + 8 gq + 4 hh .. +3 of the half (c = 0, 1)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        pv_fence(o[j][2 * hf + c]);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          *(f32x4_t*)(ep + l32 * kEpRow + 32 * c + 8 * gq + 4 * hh) =
              f32x4_t{o[j][2 * hf + c][4 * gq] * f_new, o[j][2 * hf + c][4 * gq + 1] * f_new,
                      o[j][2 * hf + c][4 * gq + 2] * f_new, o[j][2 * hf + c][4 * gq + 3] * f_new};
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // s_waitcnt lgkmcnt(0): this wave's rows are in LDS
      __builtin_amdgcn_wave_barrier();
      // lane: row 8 k + lane / 8, columns 8 (lane % 8) .. +7 of the half
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + (lane >> 3), cc = 8 * (lane & 7);
        const int qr = kQB * qb + 64 * w + 32 * j + r;
        const f32x4_t y0 = *(const f32x4_t*)(ep + r * kEpRow + cc);
        const f32x4_t y1 = *(const f32x4_t*)(ep + r * kEpRow + cc + 4);
        float y[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
        if (qr < Sq) {
          const int64_t tr = (int64_t)q0 + qr;
          uint16_t* dst = a.o + tr * a.o_s_tok + (int64_t)h * a.o_s_head + 64 * hf + cc;
          if (a.prev_o) {  // read before this lane's own write of the same 16 bytes (o may alias prev_o)
            const float fp = epf[r];
            const u32x4_t pv4 = *(const u32x4_t*)(a.prev_o + tr * a.o_s_tok + (int64_t)h * a.o_s_head + 64 * hf + cc);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              y[2 * d] += fp * bf16_to_f32((uint16_t)(pv4[d] & 0xFFFF));
              y[2 * d + 1] += fp * bf16_to_f32((uint16_t)(pv4[d] >> 16));
            }
          }
          *(u32x4_t*)dst = u32x4_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                                   pack_bf16x2(y[6], y[7])};
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads are done before the next half overwrites
      __builtin_amdgcn_wave_barrier();
    }
  }
  }  // pass
}

// Context gather: one wave per output row.  Row r belongs to the request b with
// cu[b] <= r < cu[b+1] and is context position starts[b] + r - cu[b] of that request,
// read through its block-table row.  fp8 rows are widened and multiplied by kv_scale,
// then rounded to bf16 (gather_and_maybe_dequant_cache).
template <bool FP8>
__global__ __launch_bounds__(256) void gather_ctx_kernel(GatherArgs a) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (r >= a.total) return;
  int lo = 0, hi = a.B;  // last b with cu[b] <= r
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu[mid] <= r) lo = mid;
    else hi = mid;
  }
  const int b = lo;
  const int pos = a.starts[b] + (int)(r - a.cu[b]);
  const int64_t page = a.block_table[(int64_t)b * a.bt_s + pos / a.page_size];
  const int64_t base = page * a.s_page + (int64_t)(pos % a.page_size) * a.s_tok;
  uint16_t* okv = a.out_kv_c + r * a.okv_s;
  uint16_t* ope = a.out_k_pe + r * a.ope_s;
  if constexpr (!FP8) {
    const uint16_t* kv = (const uint16_t*)a.kv_c + base;
    *(u32x4_t*)(okv + 8 * l) = *(const u32x4_t*)(kv + 8 * l);
    if (l < 8) *(u32x4_t*)(ope + 8 * l) = *(const u32x4_t*)((const uint16_t*)a.k_pe + base + 8 * l);
  } else {
    auto widen = [&](const uint8_t* src, uint16_t* dst) __attribute__((always_inline)) {
      const u32x2_t raw = *(const u32x2_t*)src;
      u32x4_t out;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const u32x2_t wb = fp8x4_to_bf16x4(raw[k]);  // exact
#pragma unroll
        for (int p = 0; p < 2; ++p)
          out[2 * k + p] = pack_bf16x2(bf16_to_f32((uint16_t)(wb[p] & 0xFFFF)) * a.kv_scale,
                                       bf16_to_f32((uint16_t)(wb[p] >> 16)) * a.kv_scale);
      }
      *(u32x4_t*)dst = out;
    };
    widen((const uint8_t*)a.kv_c + base + 8 * l, okv + 8 * l);
    if (l < 8) widen((const uint8_t*)a.k_pe + base + 8 * l, ope + 8 * l);
  }
}

}  // namespace

hipError_t launch_prefill_attn(const PrefillAttnArgs& a, int32_t B, int32_t max_q, hipStream_t stream) {
  if (B == 0 || max_q == 0) return hipSuccess;
  PrefillAttnArgs g = a;
  g.q_blocks = (max_q + kQB - 1) / kQB;
  g.items = (a.causal ? (g.q_blocks + 1) / 2 : g.q_blocks) * a.N * B;
  g.per_xcd = (g.items + 7) / 8;
  hipLaunchKernelGGL(prefill_attn_pipe_kernel, dim3(8 * g.per_xcd), dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_gather_ctx(const GatherArgs& a, bool fp8, hipStream_t stream) {
  if (a.total == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.total + 3) / 4));
  if (fp8) hipLaunchKernelGGL(gather_ctx_kernel<true>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(gather_ctx_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
