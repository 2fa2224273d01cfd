// Paged latent-MQA decode kernel for gfx950.
//
// Computes, for every query row of every request, softmax attention over the
// request's cache rows [kv_c | k_pe] with value kv_c (vLLM mla/common.py module
// docstring, "Data-Movement Friendly Approach"): an MQA whose single KV head is the
// 576-wide latent row, shared by all Sq*N query rows of the request.
//
// Work split.  One workgroup (4 waves, one per SIMD) per (plan part, head group of up
// to 128 query rows).  Wave w owns query rows 32w..32w+31: their queries stay in VGPRs
// for a whole segment, O (32 rows x 512 columns, fp32) in the 256 AGPRs.  Only the key
// tile (32 cache rows) is shared, through LDS.  The head groups of one part are dealt to
// one XCD, so when Sq*N > 128 a tile one group reads from HBM reaches the others from
// that XCD's L2.  The pipelined step loop and the stage layout are described with the
// kernel below.
//
// MFMAs (v_mfma_f32_32x32x16_bf16) are inline asm: only then does the compiler leave
// all accumulation registers to O.  It does not model MFMA hazards across inline asm,
// so the statements carry their own wait states where a VALU result or read is near:
// 3 before an MFMA whose operands a VALU may just have written, 16 after the last MFMA
// of a chain whose result is read next (the compiler itself pads 1-2 and 12 on gfx950).
#include <utility>

#include "common.h"
#include "kernels.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace mla {

namespace {

constexpr int kTile = 32;                    // keys per tile
constexpr int kStages = 4;                   // bf16 stages (bf16 caches)
constexpr int kRowB = 1168;                  // LDS bytes per key row (576 bf16 + 16 pad)
constexpr int kRowC = kRowB / 16;            // 73 chunks
constexpr int kStageB = kTile * kRowB;       // 37376
constexpr int kStageC = kTile * kRowC;       // 2336
constexpr int kDmaN = (kStageC + 63) / 64;   // 37 DMA instructions per tile
static_assert(kDmaN == 37, "the last DMA instruction of a tile is the only partial one");
constexpr int kSmemBytes = kStages * kStageB;  // 149504
constexpr float kRescaleAt = 8.f;  // log2 units a tile maximum may exceed the reference by

// fp8 queries (fp8 cache only): raw e4m3 tiles, read as they are by the fp8 QK, in a
// 4-slot ring; the value columns of each tile are widened into one of two bf16 stages
// (the stage layout above, rope columns unused) for the bf16 P.V.
constexpr int kQRowB = 592;                    // raw row: 576 bytes + 16 pad
constexpr int kQRowC = kQRowB / 16;            // 37 chunks (odd: conflict-free reads)
constexpr int kQSlotB = kTile * kQRowB;        // 18944
constexpr int kQSlots = 4;
constexpr int kQVBase = kQSlots * kQSlotB;     // 75776: the two value stages follow
constexpr int kQSmem = kQVBase + 2 * kStageB;  // 150528
constexpr int kSmemAll = kQSmem > kSmemBytes ? kQSmem : kSmemBytes;

__shared__ __attribute__((aligned(1024))) char smem[kSmemAll];

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// HBM -> LDS, 16 bytes per lane: lane l writes LDS bytes [m0 + 16 l, m0 + 16 l + 16).
// 64-bit per-lane address.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
// Waits until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// A tile is PER DMA instructions per wave; waits until at most `newer` tiles issued
// after the awaited one are pending (vector-memory loads complete in issue order).
template <int PER>
__device__ __forceinline__ void wait_tiles(int newer) {
  switch (newer) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<PER>(); break;
    case 2: wait_vm<2 * PER>(); break;
    default: wait_vm<3 * PER>(); break;
  }
}
// The same wait in the step loop, where `newer` is 1 but for a segment's first steps and
// a part's last ones: with newer >= 1 it leaves MIN (the fewest DMA instructions any wave
// issues per tile) loads outstanding, which waits for at least the awaited tile, and the
// branch stays two adjacent blocks (a switch laid out away from the loop cost each step
// a few hundred cycles of jumps there and back).
template <int MIN>
__device__ __forceinline__ void wait_landed(int newer) {
  if (newer > 0) wait_vm<MIN>();
  else wait_vm<0>();
}
// Workgroup barrier that also orders this wave's LDS accesses (and does not drain vmcnt).
// The lgkmcnt(0) wait is the compiler's own, so it knows that every LDS and scalar load
// issued before is complete and places no conservative waits after the barrier.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // s_waitcnt lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// ---- MFMA statements (see the header for the wait states) ----
__device__ __forceinline__ void mfma_acc_v(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_v_last(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7" : "+v"(d) : "v"(a), "v"(b));
}
// Orders VALU writes of an accumulator before the next MFMA that reads it.
__device__ __forceinline__ void acc_written(f32x16_t& d) { asm volatile("s_nop 2" : "+a"(d)); }
// Zeroes the 16 output accumulators in place (0 * 0 + 0 on the MFMA unit), without a
// zero vector in VGPRs that the compiler would keep live across the loops.
template <int NB>
__device__ __forceinline__ void acc_zero(f32x16_t (&o)[NB]) {
  u32x4_t z;  // made here, so that no zero vector stays live (or spilled) across the loops
  asm volatile("v_mov_b32 %0, 0\n\tv_mov_b32 %1, 0\n\tv_mov_b32 %2, 0\n\tv_mov_b32 %3, 0"
               : "=v"(z[0]), "=v"(z[1]), "=v"(z[2]), "=v"(z[3]));
#pragma unroll
  for (int i = 0; i < NB - 1; ++i)
    asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=&a"(o[i]) : "v"(z));
  // an empty segment reads the accumulators right away
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0\n\ts_nop 7\n\ts_nop 7" : "=&a"(o[NB - 1])
               : "v"(z));
}
// 16-byte global load that the compiler does not track: the caller waits for it with an
// explicit vmcnt and reads the destination only after that wait.
template <int OFF>
__device__ __forceinline__ void gload16(u32x4_t& d, const void* p) {
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2 ; qload" : "=v"(d) : "v"(p), "n"(OFF) : "memory");
}
// Lane index, recomputed where it is used: values derived from it (query and output
// addresses) are then rebuilt at each segment instead of held in VGPRs across the tile
// loop, where the register allocator would spill them; a spill reload is a vector-memory
// load, and waiting for it would drain the DMA loads in flight.
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
// Keeps an accumulator in AGPRs up to this point, so that the compiler copies it to
// VGPRs only where it is read, one block at a time (not all 256 registers at once).
__device__ __forceinline__ void acc_fence(f32x16_t& d) { asm volatile("" : "+a"(d)::"memory"); }

struct Seg {
  int b, ks, ke, pidx;
};
__device__ __forceinline__ Seg load_seg(const int32_t* segs, int si) {
  return Seg{ld_uniform(segs + 4 * si), ld_uniform(segs + 4 * si + 1), ld_uniform(segs + 4 * si + 2),
             ld_uniform(segs + 4 * si + 3)};
}

// Tile cursor over the part's segments: segment index, first key of the tile, and the
// segment's request and key end (kept so that advancing needs no loads within a segment).
struct Cursor {
  int si, ts, b, ke;
};
__device__ __forceinline__ Cursor first_tile(const int32_t* segs, int si, int s_end) {
  for (; si < s_end; ++si) {
    const Seg s = load_seg(segs, si);
    if (s.ke > s.ks) return Cursor{si, s.ks, s.b, s.ke};
  }
  return Cursor{s_end, 0, 0, 0};
}
__device__ __forceinline__ Cursor next_tile(const int32_t* segs, Cursor c, int s_end) {
  if (c.ts + kTile < c.ke) return Cursor{c.si, c.ts + kTile, c.b, c.ke};
  return first_tile(segs, c.si + 1, s_end);
}

// Byte offset (from the cache base) of key row j of a request, for a wave-uniform j
// (scalar block_table load); esz = element size.
__device__ __forceinline__ int64_t row_bytes(const DecodeArgs& a, const int32_t* bt_row, int j, int esz) {
  const unsigned ps = (unsigned)a.page_size;
  const int page = ld_uniform(bt_row + (unsigned)j / ps);
  return ((int64_t)page * a.s_page + (int64_t)((unsigned)j % ps) * a.s_tok) * esz;
}

// Wave-uniform description of one tile's DMA.  With pages of a multiple of 32 keys the
// tile sits in one page: one block_table lookup gives its base, then 32-bit offsets.
struct DmaTile {
  const char* kv;  // PAGED32: cache base + byte offset of the tile's first key; else cache base
  const char* pe;
  const int32_t* bt_row;
  int ts, kmax;  // first key, last valid key offset within the tile
  uint32_t lds;  // bf16 stage or raw fp8 stage
};

template <bool FP8, bool PAGED32>
__device__ __forceinline__ DmaTile dma_tile(const DecodeArgs& a, const Cursor& pf, uint32_t lds) {
  DmaTile t;
  t.bt_row = a.block_table + (int64_t)pf.b * a.bt_s;
  t.ts = pf.ts;
  t.kmax = pf.ke - pf.ts - 1;
  t.lds = lds;
  const int64_t tb = PAGED32 ? row_bytes(a, t.bt_row, pf.ts, FP8 ? 1 : 2) : 0;
  t.kv = (const char*)a.kv_c + tb;
  t.pe = (const char*)a.k_pe + tb;
  return t;
}

// 8 bf16 of V^T (column of this lane, 8 keys) from the row-major tile: two transposing
// reads of 4 keys each (p0: elements 0..3 of the MFMA operand, p1: elements 4..7).
__device__ __forceinline__ u32x4_t read_vt(const char* p0, const char* p1) {
  const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const lds_char*)p0);
  const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const lds_char*)p1);
  const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0), w1 = __builtin_bit_cast(u32x2_t, v1);
  return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
}

}  // namespace

// ---------------------------------------------------------------------------------
// Software-pipelined decode kernel.  Wave w owns query rows 32w..32w+31 from end to end:
// Q in VGPRs, O (all 512 columns) in the 256 AGPRs and P in VGPRs, so only the key tile
// is shared.  Step s of a segment of n tiles (s = 0..n):
//   wait for tile s, barrier;
//   QK of tile s (36 MFMAs), with this wave's DMA of a later tile between its MFMAs;
//   P.V of tile s-1 (32 MFMAs), with the softmax of tile s between them;
//   rescale of O when tile s raised a row's reference maximum (rare).
// One loop body serves every step, so O stays in one set of registers: step 0 runs its
// P.V with P = 0 against the landed tile 0, and step n has no QK (its softmax sees every
// key masked).  A stage is reloaded once the P.V of the tile it held is complete, two
// steps before its QK.  fp8 caches add a widening of each tile to bf16 one step ahead
// (see the fp8 ring below).
// With one wave per SIMD every instruction takes an issue slot of the MFMA stream, so
// the per-tile address and bookkeeping work is kept small.
//
// Stage layout: key row k of the tile (576 bf16, latent then rope) at k * 1168 bytes,
// a 16-byte pad after each row.  The odd 16-byte shift between rows (73 chunks) keeps
// both read patterns free of bank conflicts (64 banks of 4 bytes; a 16-byte chunk's
// bank group is its index mod 16) with addresses that are affine in the k-step:
//  QK   ds_read_b128: S^T row i of the MFMA holds key pi(i) = ((i>>2)&3) + 4(i&3) +
//       16(i>>4), a bijection that gives the 16 lanes of one access 16 keys with
//       distinct residues mod 16, hence 16 distinct bank groups for the same chunk;
//  P.V  ds_read_b64_tr_b16: with that order the 4 keys of one transposing read are
//       {x, x+4, x+8, x+12}, 4 * 73 = 4 mod 16 bank groups apart, and each spans 4
//       consecutive groups.
// A tile is 2336 chunks, written by 37 DMA instructions of 1 KB (the last one half),
// the pads receiving a copy of a neighbouring chunk.
// ---------------------------------------------------------------------------------


// Calls f(std::integral_constant<int, K>) for K = 0..N-1 in order, as straight-line code.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... K>(std::integer_sequence<int, K...>) {
    (f(std::integral_constant<int, K>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}

// Marks a value as (re)defined here: work that uses it cannot move above this point.
template <typename T>
__device__ __forceinline__ void redef(T& x) { asm volatile("" : "+v"(x)); }
// Marks a value as used here: the work producing it cannot move below this point.
template <typename T>
__device__ __forceinline__ void use(const T& x) { asm volatile("" ::"v"(x)); }

// MFMAs whose A/B operands come from LDS or were written many instructions earlier
// (no VALU write of them can sit right before): no leading wait states.
__device__ __forceinline__ void mfma_v_first_nw(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_a_nw(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}

// fp8 x fp8 MFMA (v_mfma_f32_32x32x64_f8f6f4, both operands e4m3, 16 passes): D += A B
// over 64 k.  Lane l holds A[l%32][k] and B[k][l%32] for 32 values of k in the lane
// half l/32; which 32 is the same for A and B, so a contraction only needs both operands
// loaded alike.  The last of a chain pads the 18 wait states a VALU read of D needs.
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ u32x8_t cat8(const u32x4_t& lo, const u32x4_t& hi) {
  return u32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ void mfma8_first(f32x16_t& d, const u32x8_t& a, const u32x8_t& b) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma8_acc(f32x16_t& d, const u32x8_t& a, const u32x8_t& b) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma8_last(f32x16_t& d, const u32x8_t& a, const u32x8_t& b) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d)
               : "v"(a), "v"(b));
}

// HBM -> LDS, 16 bytes per lane at lds_base + IMM + 16 lane, from gbase + voff.
template <int IMM>
__device__ __forceinline__ void dma16_si(const void* gbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase),
               "s"(lds_base), "n"(IMM)
               : "memory", "m0", "scc");
}


// Softmax ops as volatile statements, so that each stays in the slot between two MFMAs
// where it is written (the compiler keeps volatile statements in order).  Their operands
// come from ops at least one MFMA earlier, which also covers the one wait state a
// transcendental result needs before its use.
__device__ __forceinline__ void vmax3(float& d, float a, float b, float c) {
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
}
__device__ __forceinline__ void vfma(float& d, float a, float b, float c) {
  asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(b), "v"(c));
}
__device__ __forceinline__ void vexp2(float& d, float a) { asm volatile("v_exp_f32 %0, %1" : "=v"(d) : "v"(a)); }
__device__ __forceinline__ void vadd(float& d, float a, float b) {
  asm volatile("v_add_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void vcvt_bf16x2(uint32_t& d, float lo, float hi) {
  asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(d) : "v"(lo), "v"(hi));
}
// d += lo + hi of a packed bf16 pair (a dot product with the pair (1, 1)): a row sum of
// exactly the rounded probabilities that the P.V MFMAs multiply.  A builtin, not a
// scheduled statement: the compiler places it and keeps the wait states it needs.
constexpr uint32_t kBf16Ones = 0x3F803F80u;
__device__ __forceinline__ void dot2_sum(float& d, uint32_t pk) {
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), __builtin_bit_cast(bf16x2_t, kBf16Ones), d,
                                      false);
}

// Tile key (0..31) held by S^T accumulator row i.
__device__ __forceinline__ int row_key(int i) { return ((i >> 2) & 3) + 4 * (i & 3) + 16 * (i >> 4); }

// fp8 caches: 3 bf16 stages, then a ring of raw e4m3 tiles: wave w owns two slots of
// 8 rows x 576 bytes (the rows it loads and widens).
constexpr int kRawWaveTile = 8 * kHead;       // 4608
constexpr int kRawBase = 3 * kStageB;         // 112128
static_assert(kRawBase + 4 * 2 * kRawWaveTile <= kSmemBytes, "fp8 stages fit");

// FAST: pages of a multiple of 32 keys (a tile sits in one page) and the rope columns
// right after the latent ones in each cache row (one base for the whole row).
// FP8: e4m3 cache, widened to bf16 in LDS (every e4m3 value is exact in bf16).
// QF8 (with FP8): e4m3 queries; QK on the fp8 MFMA over the raw tile, only the value
// columns widened to bf16 for P.V.
template <bool FAST, bool FP8, bool QF8>
__global__ __launch_bounds__(256, 1) void mla_decode_pipe_kernel(DecodeArgs a) {
  static_assert(!QF8 || FP8, "fp8 queries go with an fp8 cache");
  constexpr bool RAWW = FP8 && !QF8;  // fp8 cache widened whole, per-wave raw ring
  // K fragment ring depth, and DMA steps issued before the first QK MFMA (they fill the
  // wait for the first fragments); chosen by measurement on the DSV3 and verify shapes
  constexpr int KRING = 6, DMA0 = 2;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in an SGPR
  const int lane = tid & 63, r32 = lane & 31, h2 = lane >> 5;

  // Workgroups are dealt round-robin to the 8 XCDs.  XCD x takes a contiguous range of
  // ceil(parts / 8) parts, so the parts of one request (consecutive in the plan) mostly
  // share an XCD's L2 for their queries, and the head groups of one part share it for
  // the part's keys.
  const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const int hg = slot % a.head_groups;
  const int part = xcd * ((a.num_parts + 7) / 8) + slot / a.head_groups;
  if (part >= a.num_parts) return;

  const int R = a.Sq * a.N;
  const int row0 = hg * kGroupRows;
  const int RG = min(kGroupRows, R - row0);  // rows of this group
  const bool has_rows = 32 * w < RG;         // wave-uniform
  // token t and head h of this lane's row 32w + l%32 of the group: the division is done
  // once per wave on uniform values, the lane's remainder by at most 32 subtractions
  // (no per-lane reciprocal held across the loops)
  const int tw = (row0 + 32 * w) / a.N, hw = (row0 + 32 * w) - tw * a.N;
  auto row_th = [&](int i, int& t, int& h) __attribute__((always_inline)) {
    t = tw;
    h = hw + i;
    while (h >= a.N) {
      h -= a.N;
      ++t;
    }
  };
  const int32_t* segs = a.segs;
  const int s_beg = ld_uniform(a.part_begin + part), s_end = ld_uniform(a.part_begin + part + 1);
  const float c = a.qk_scale_log2;
  const uint32_t st = (uint32_t)a.s_tok * (FP8 ? 1 : 2);  // bytes between cache rows
  const uint32_t smem0 = lds_addr(smem);
  constexpr int NST = FP8 ? 3 : kStages;  // bf16 stages

  // ---- DMA: wave w issues instructions j = w + 4n of a tile (n = 0..8, and n = 9 for
  // wave 0: j = 36, lanes 0..31).  Lane l of instruction j writes stage chunk p = 64j + l
  // = key p / 73, chunk p % 73 (the pad, chunk 72, takes a copy of chunk 71).
  const bool w0 = w == 0;
  auto chunk_key = [&](int n) __attribute__((always_inline)) { return (64 * (w + 4 * n) + lane) / kRowC; };
  auto chunk_col = [&](int n) __attribute__((always_inline)) {
    return min((64 * (w + 4 * n) + lane) % kRowC, kRowC - 2);
  };
  uint32_t dvo[10];  // FAST: byte offsets from the tile's first row
#pragma unroll
  for (int n = 0; n < 10; ++n) dvo[n] = (uint32_t)chunk_key(n) * st + 16u * (uint32_t)chunk_col(n);

  auto dma_one = [&](const DmaTile& t, auto nc) __attribute__((always_inline)) {
    constexpr int n = decltype(nc)::value;
    if constexpr (n == 9) {
      if (!w0 || lane >= 32) return;
    }
    if constexpr (FAST) {
      dma16_si<4096 * n>(t.kv, dvo[n], t.lds + 1024 * w);
    } else {
      // generic pages: the rows of this instruction (at most two) through the block table
      const int k0 = (64 * (w + 4 * n)) / kRowC;  // wave-uniform
      const int64_t rb0 = row_bytes(a, t.bt_row, t.ts + min(k0, t.kmax), 2);
      const int64_t rb1 = row_bytes(a, t.bt_row, t.ts + min(k0 + 1, t.kmax), 2);
      const int col = chunk_col(n);
      const int64_t rb = chunk_key(n) == k0 ? rb0 : rb1;
      const char* src = col < 64 ? (const char*)t.kv + rb + 16 * col : (const char*)t.pe + rb + 16 * (col - 64);
      dma16(src, t.lds + 1024 * (w + 4 * n));
    }
  };
  // Keys past the segment end load key kmax instead (FAST: offsets moved to row kmax
  // for the tile, dir = -1, and back, dir = +1).
  auto dma_clamp = [&](const DmaTile& t, int dir) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < 10; ++n) dvo[n] += (uint32_t)(dir * max(chunk_key(n) - t.kmax, 0)) * st;
  };
  const int wkey = (64 * w + 64 * 4 * 9 + 63) / kRowC;  // upper bound of the keys this wave loads
  auto dma_all = [&](const DmaTile& t) __attribute__((always_inline)) {
    const bool clamp = FAST && t.kmax < wkey;
    if (clamp) dma_clamp(t, -1);
    static_for<10>([&](auto nc) __attribute__((always_inline)) { dma_one(t, nc); });
    if (clamp) dma_clamp(t, 1);
  };

  // ---- fp8: wave w loads rows 8w..8w+7 of a tile as raw e4m3 into its own slot of a
  // two-tile ring and widens them into the bf16 stage one step before the QK that reads
  // them; no other wave reads the slot, so it is refilled without a barrier.  DMA
  // instruction n = 0..4 (4: lanes 0..31) covers raw chunk p = 64n + lane of the wave's
  // rows: row p / 36, 16-byte chunk p % 36.
  auto raw_row = [&](int n) __attribute__((always_inline)) { return (64 * n + lane) / 36; };
  auto raw_col = [&](int n) __attribute__((always_inline)) { return (64 * n + lane) % 36; };
  uint32_t rvo[5];  // FAST: byte offsets from the tile's first row
#pragma unroll
  for (int n = 0; n < 5; ++n) rvo[n] = (uint32_t)(8 * w + raw_row(n)) * st + 16u * (uint32_t)raw_col(n);
  auto raw_slot = [&](int gi) __attribute__((always_inline)) {
    return smem0 + kRawBase + (uint32_t)(2 * w + (gi & 1)) * kRawWaveTile;
  };
  auto dma_raw = [&](const DmaTile& t) __attribute__((always_inline)) {
    const bool clamp = t.kmax < 8 * w + 7;  // wave-uniform: the tile ends inside these rows
    static_for<5>([&](auto nc) __attribute__((always_inline)) {
      constexpr int n = decltype(nc)::value;
      if constexpr (n == 4) {
        if (lane >= 32) return;
      }
      if constexpr (FAST) {
        uint32_t off = rvo[n];
        if (clamp) off -= (uint32_t)max(8 * w + raw_row(n) - t.kmax, 0) * st;
        dma16_si<1024 * n>(t.kv, off, t.lds);
      } else {
        // generic pages: the rows of this instruction (at most three) through the block table
        const int k0 = 8 * w + (64 * n) / 36;  // wave-uniform
        const int64_t rb0 = row_bytes(a, t.bt_row, t.ts + min(k0, t.kmax), 1);
        const int64_t rb1 = row_bytes(a, t.bt_row, t.ts + min(k0 + 1, t.kmax), 1);
        const int64_t rb2 = row_bytes(a, t.bt_row, t.ts + min(k0 + 2, t.kmax), 1);
        const int kr = 8 * w + raw_row(n) - k0, col = raw_col(n);
        const int64_t rb = kr == 0 ? rb0 : (kr == 1 ? rb1 : rb2);
        const char* src = col < 32 ? (const char*)t.kv + rb + 16 * col : (const char*)t.pe + rb + 16 * (col - 32);
        dma16(src, t.lds + 1024 * n);
      }
    });
  };
  // Widens chunk i of this wave's raw rows (slot `raw`, LDS address) into the bf16 stage
  // at byte offset `dst` of smem: i < 8 is row i, values 8 lane .. +7 (latent); i = 8 is
  // row lane / 8, rope values 8 (lane % 8) .. +7.  Read and conversion are separate
  // steps, so that all 9 reads of a tile can be in flight at once.
  auto widen_rd = [&](uint32_t raw, auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    const int ln = i < 8 ? lane : lane_now();  // (i = 8: no lane offset kept live for it)
    const int row = i < 8 ? i : (ln >> 3);
    const int col8 = i < 8 ? ln : 64 + (ln & 7);
    return *(const u32x2_t*)(smem + (raw - smem0) + row * kHead + 8 * col8);
  };
  auto widen_wr = [&](uint32_t dst, auto ic, const u32x2_t& v) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    const int ln = i < 8 ? lane : lane_now();
    const int row = i < 8 ? i : (ln >> 3);
    const int col8 = i < 8 ? ln : 64 + (ln & 7);
    const u32x2_t lo = fp8x4_to_bf16x4(v[0]), hi = fp8x4_to_bf16x4(v[1]);
    *(u32x4_t*)(smem + dst + (8 * w + row) * kRowB + 16 * col8) = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  };
  auto widen = [&](uint32_t raw, uint32_t dst, auto ic) __attribute__((always_inline)) {
    widen_wr(dst, ic, widen_rd(raw, ic));
  };
  // The whole tile: the 9 reads issued together, then the conversions and writes, each
  // after its own read (the compiler pairs the reads and waits for them in order).
  auto widen_all = [&](uint32_t raw, uint32_t dst) __attribute__((always_inline)) {
    u32x2_t v[9];
    static_for<9>([&](auto ic) __attribute__((always_inline)) { v[decltype(ic)::value] = widen_rd(raw, ic); });
    static_for<9>([&](auto ic) __attribute__((always_inline)) { widen_wr(dst, ic, v[decltype(ic)::value]); });
  };

  // ---- fp8 queries: all waves load each raw tile into its slot of the 4-slot ring: wave
  // w issues instructions j = w + 4n (n = 0..4, j < 19; j = 18: lanes 0..31).  Lane l of
  // instruction j writes slot chunk p = 64j + l = row p / 37, chunk p % 37 (the pad, chunk
  // 36, takes a copy of chunk 35).  A tile is PERQ = 5 (wave 3: 4) instructions per wave.
  auto q8_row = [&](int n) __attribute__((always_inline)) { return (64 * (w + 4 * n) + lane) / kQRowC; };
  auto q8_col = [&](int n) __attribute__((always_inline)) {
    return min((64 * (w + 4 * n) + lane) % kQRowC, kQRowC - 2);
  };
  uint32_t qvo[5];  // FAST: byte offsets from the tile's first row
  if constexpr (QF8) {
#pragma unroll
    for (int n = 0; n < 5; ++n) qvo[n] = (uint32_t)q8_row(n) * st + 16u * (uint32_t)q8_col(n);
  }
  const int qwkey = (64 * (w + 16) + 63) / kQRowC;  // upper bound of the rows this wave loads
  auto dma_q8_one = [&](const DmaTile& t, auto nc) __attribute__((always_inline)) {
    constexpr int n = decltype(nc)::value;
    if constexpr (n == 4) {
      if (w == 3) return;                // j = 19: past the tile (wave-uniform)
      if (w == 2 && lane >= 32) return;  // j = 18: the tile's last 32 chunks
    }
    if constexpr (FAST) {
      dma16_si<4096 * n>(t.kv, qvo[n], __builtin_amdgcn_readfirstlane(t.lds + 1024 * w));
    } else {
      // generic pages: the rows of this instruction (at most three) through the block table
      const int k0 = (64 * (w + 4 * n)) / kQRowC;  // wave-uniform
      const int64_t rb0 = row_bytes(a, t.bt_row, t.ts + min(k0, t.kmax), 1);
      const int64_t rb1 = row_bytes(a, t.bt_row, t.ts + min(k0 + 1, t.kmax), 1);
      const int64_t rb2 = row_bytes(a, t.bt_row, t.ts + min(k0 + 2, t.kmax), 1);
      const int kr = q8_row(n) - k0, col = q8_col(n);
      const int64_t rb = kr == 0 ? rb0 : (kr == 1 ? rb1 : rb2);
      const char* src = col < 32 ? (const char*)t.kv + rb + 16 * col : (const char*)t.pe + rb + 16 * (col - 32);
      dma16(src, t.lds + 1024 * (w + 4 * n));
    }
  };
  auto dma_q8 = [&](const DmaTile& t) __attribute__((always_inline)) {
    // rows past the tile's last key load that key (FAST: offsets moved there and back)
    const bool clamp = FAST && t.kmax < qwkey;
    if (clamp) {
#pragma unroll
      for (int n = 0; n < 5; ++n) qvo[n] -= (uint32_t)max(q8_row(n) - t.kmax, 0) * st;
    }
    static_for<5>([&](auto nc) __attribute__((always_inline)) { dma_q8_one(t, nc); });
    if (clamp) {
#pragma unroll
      for (int n = 0; n < 5; ++n) qvo[n] += (uint32_t)max(q8_row(n) - t.kmax, 0) * st;
    }
  };
  // Value columns of this wave's rows 8w..8w+7 of a raw tile, widened into a bf16 value
  // stage: lane l takes row 8w + l%8, bytes 64(l/8) .. +63 (four 16-byte reads, eight
  // 16-byte writes; part i = 0..3 converts read i).
  const uint32_t q8wsrc = (uint32_t)(8 * w + (lane & 7)) * kQRowB + 64 * (lane >> 3);
  const uint32_t q8wdst = (uint32_t)(8 * w + (lane & 7)) * kRowB + 128 * (lane >> 3);
  auto widen8_read = [&](uint32_t slot, u32x4_t (&wr)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[i] = *(const u32x4_t*)(smem + slot + q8wsrc + 16 * i);
  };
  auto widen8_part = [&](uint32_t vstage, const u32x4_t (&wr)[4], int i) __attribute__((always_inline)) {
    const u32x2_t b0 = fp8x4_to_bf16x4(wr[i][0]), b1 = fp8x4_to_bf16x4(wr[i][1]);
    const u32x2_t b2 = fp8x4_to_bf16x4(wr[i][2]), b3 = fp8x4_to_bf16x4(wr[i][3]);
    *(u32x4_t*)(smem + vstage + q8wdst + 32 * i) = u32x4_t{b0[0], b0[1], b1[0], b1[1]};
    *(u32x4_t*)(smem + vstage + q8wdst + 32 * i + 16) = u32x4_t{b2[0], b2[1], b3[0], b3[1]};
  };
  // fp8 QK A operand: key row_key(r32) of the raw tile, 32 bytes of k-step c at +64c
  const uint32_t kq8base = (uint32_t)row_key(r32) * kQRowB + 32 * h2;

  // ---- LDS read addresses (bytes from a stage base) ----
  // QK A operand: key row_key(r32), logical chunk 2k + h2 at kbase + 32 k.
  const uint32_t kbase = (uint32_t)row_key(r32) * kRowB + 16 * h2;
  // P.V A operand through ds_read_b64_tr_b16 (16-lane group g covers columns 32cb +
  // 16(g & 1) + 0..15; lane j addresses key x + 4(j >> 2) at columns +4(j & 3) and
  // receives those 4 keys of column +j): for k-step s the keys are x = h2 + 16s (e = 0..3)
  // and x + 2 (e = 4..7), matching the B operand P^T = elements 8s..8s+7 of S^T.
  const uint32_t vbase = (uint32_t)(h2 + 4 * ((lane & 15) >> 2)) * kRowB + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

  // ---- queries: the B operand of S^T = K . Q^T, 36 x 8 bf16 per lane (lane: row 32w +
  // l%32 of the group, dims 16k + 8(l/32) .. +7 of k-step k).  Loaded ahead of use by
  // untracked loads (the first segment's before the DMA prologue, each later one in the
  // last step of the segment before) and waited for with a vmcnt that leaves the DMA
  // loads issued after them in flight.  Padding rows load the wave's last row and are
  // zeroed once loaded (zero queries give zero logits; their rows are never stored).
  // fp8 queries: 9 k-steps of 64 dims, 32 bytes per lane (dims 64c + 32(l/32) .. +31)
  // in qr[2c], qr[2c + 1].
  constexpr int NQ = QF8 ? 18 : 36;
  u32x4_t qr[NQ];
  auto issue_q = [&](int b) __attribute__((always_inline)) {
    const int ln = lane_now();
    int t, h;
    row_th(min(ln & 31, RG - 1 - 32 * w), t, h);
    const int64_t tok = (int64_t)b * a.Sq + t;
    if constexpr (QF8) {
      const uint8_t* q8 = a.q8 + tok * a.q8_s_tok + (int64_t)h * a.q8_s_head + 32 * (ln >> 5);
      static_for<18>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        gload16<64 * (k >> 1) + 16 * (k & 1)>(qr[k], q8);
      });
    } else {
      const uint16_t* qn = a.q_nope + tok * a.q_nope_s_tok + (int64_t)h * a.q_nope_s_head + 8 * (ln >> 5);
      const uint16_t* qp = a.q_pe + tok * a.q_pe_s_tok + (int64_t)h * a.q_pe_s_head + 8 * (ln >> 5);
      static_for<32>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        gload16<32 * k>(qr[k], qn);
      });
      static_for<4>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        gload16<32 * k>(qr[32 + k], qp);
      });
    }
  };
  auto q_landed = [&]() __attribute__((always_inline)) {
    if (32 * w + 32 > RG) {  // wave-uniform: the wave has padding rows
      const bool pad = 32 * w + (lane_now() & 31) >= RG;
#pragma unroll
      for (int k = 0; k < NQ; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) qr[k][e] = pad ? 0u : qr[k][e];
    }
  };
  if (has_rows && s_beg < s_end) issue_q(ld_uniform(segs + 4 * s_beg));

  Cursor pf = first_tile(segs, s_beg, s_end);  // next tile to load
  int issued = 0, done = 0;                    // tiles issued; tiles of finished segments
  int widened = 0;                             // fp8: tiles widened into their bf16 stage
  if constexpr (QF8) {
    // raw tiles 0..2; the value stages start at zero (the first step of a segment
    // multiplies P = 0 by the stage of the tile before, which must hold finite values)
#pragma unroll 1
    for (int k = 0; k < 3; ++k) {
      if (pf.si >= s_end) break;
      dma_q8(dma_tile<true, FAST>(a, pf, smem0 + (issued % kQSlots) * kQSlotB));
      pf = next_tile(segs, pf, s_end);
      issued++;
    }
#pragma unroll 1
    for (int i = tid; i < 2 * kStageB / 16; i += 256) *(u32x4_t*)(smem + kQVBase + 16 * i) = u32x4_t{0, 0, 0, 0};
  } else if constexpr (RAWW) {
    // raw tiles 0 and 1, tile 0 widened into stage 0, raw tile 2 into the freed slot
#pragma unroll 1
    for (int k = 0; k < 2; ++k) {
      if (pf.si >= s_end) break;
      dma_raw(dma_tile<true, FAST>(a, pf, raw_slot(issued)));
      pf = next_tile(segs, pf, s_end);
      issued++;
    }
    if (issued > 0) {
      if (issued > 1) wait_vm<5>();
      else wait_vm<0>();
      static_for<9>([&](auto ic) __attribute__((always_inline)) { widen(raw_slot(0), 0, ic); });
      widened = 1;
      if (pf.si < s_end) {
        dma_raw(dma_tile<true, FAST>(a, pf, raw_slot(issued)));
        pf = next_tile(segs, pf, s_end);
        issued++;
      }
    }
  } else {
    // tiles 0 and 1 only: every workgroup starts by loading 147 KB of queries, and the
    // start-up burst of all workgroups is what the first step waits for; the steps load
    // one tile each from then on, two ahead of the QK, as in the steady state
#pragma unroll 1
    for (int k = 0; k < 2; ++k) {
      if (pf.si >= s_end) break;
      const DmaTile t = dma_tile<false, FAST>(a, pf, smem0 + (issued % kStages) * kStageB);
      dma_all(t);
      pf = next_tile(segs, pf, s_end);
      issued++;
    }
  }
  if (has_rows && s_beg < s_end) {
    // the first queries were issued before every DMA load
    if constexpr (QF8) {
      if (w == 3) wait_tiles<4>(issued);
      else wait_tiles<5>(issued);
    } else if constexpr (RAWW) {
      wait_vm<5>();
    } else {
      if (w0) wait_tiles<10>(issued);
      else wait_tiles<9>(issued);
    }
    q_landed();
  }

  for (int si = s_beg; si < s_end; ++si) {
    const Seg sg = load_seg(segs, si);
    const int b = sg.b, ks = sg.ks, ke = sg.ke, pidx = sg.pidx;
    const int L = ld_uniform(a.seq_lens + b);
    const int nt = (ke - ks + kTile - 1) / kTile;
    // keys j < lim are visible to this lane's row (segment end, causal window); every
    // row sees at least the keys below lim_lo (wave-uniform)
    const int lim_lo = min(ke, L - a.Sq + 1);
    int lim = ke;

    if (has_rows) {
      int t, h;
      row_th(lane_now() & 31, t, h);
      lim = min(ke, L - (a.Sq - 1) + t);
    }
    const bool more = si + 1 < s_end;
    bool dma_last = false;  // a DMA was issued in the last step (after the next queries)

    float m_ref = -INFINITY;  // reference maximum of this lane's row (log2 units)
    float nm = 0.f;           // exponent offset: -m_ref (0 while m_ref = -inf)
    float thr = -INFINITY;    // (m_ref + 8) / c: elements of S above it need a new reference
    float l_acc = 0.f;        // running sum over this lane's 16 keys of each tile
    float l_rnd = 0.f;        // the same sum over the bf16-rounded probabilities
    f32x16_t O[16];           // O^T[32 cols of block cb][32 rows], in AGPRs
    acc_zero<16>(O);
    f32x16_t sc;              // S^T of the tile in QK
    // P of the previous tile as bf16 pairs: the B operands of its two P.V k-steps
    u32x4_t pq[2] = {u32x4_t{0, 0, 0, 0}, u32x4_t{0, 0, 0, 0}};

    // (an empty request's segment has no tiles: no steps, and the epilogue writes o = 0,
    // lse = -inf; the DMA cursor skips such segments)
    const int g0 = done;  // part-wide index of the segment's first tile
#pragma unroll 1
    for (int s = 0; s <= nt && nt > 0; ++s) {
      const int g = g0 + s;  // part-wide index of tile s (its stage is g % kStages)
      const bool first = s == 0, last = s == nt;
      // ---- wait for tile s, decide the DMA of this step, barrier ----
      bool do_dma;
      DmaTile dt{};
      // fp8: tile s was widened before; this step widens tile s+1 (once: the last step of
      // a segment and the first of the next have the same s) into the stage of tile s-2,
      // then loads the next raw tile into the slot that frees
      const bool widen_next = RAWW && widened == g + 1 && widened < issued;  // wave-uniform
      if constexpr (QF8) {
        if (!last) wait_landed<4>(issued - g - 1);  // this wave's part of tile s has landed
        // raw slot of tile g-1 is free after this barrier: tiles up to g+3 may be in flight
        do_dma = pf.si < s_end && issued < g + kQSlots;
        if (do_dma) dt = dma_tile<true, FAST>(a, pf, smem0 + ((unsigned)issued % kQSlots) * kQSlotB);
      } else if constexpr (RAWW) {
        do_dma = pf.si < s_end && issued < widened + (widen_next ? 3 : 2);
        if (do_dma) dt = dma_tile<true, FAST>(a, pf, raw_slot(issued));
      } else {
        if (!last) wait_landed<9>(issued - g - 1);  // this wave's part of tile s has landed
        // a stage is free once the P.V of its tile is complete: before this barrier, every
        // tile up to g-2 (g-1 at the segment's first step)
        do_dma = pf.si < s_end && issued < g + (first ? kStages : kStages - 1);
        if (do_dma) dt = dma_tile<false, FAST>(a, pf, smem0 + ((unsigned)issued % kStages) * kStageB);
      }
      barrier_lds();  // tile s is in its stage for every wave; the stage of tile s-2 is free
      // QK stage (QF8: raw slot of tile g), P.V stage, stage the widening writes (QF8: the
      // value stage of tile g, read by the P.V of the next step)
      const uint32_t qst = QF8 ? ((unsigned)g % kQSlots) * kQSlotB : ((unsigned)(last ? g - 1 : g) % NST) * kStageB;
      const uint32_t pst = QF8 ? kQVBase + ((unsigned)(g - 1) & 1u) * kStageB
                               : ((unsigned)(first ? g : g - 1) % NST) * kStageB;
      const uint32_t wst = QF8 ? kQVBase + ((unsigned)g & 1u) * kStageB : ((unsigned)(g + 1) % NST) * kStageB;
      auto raw_ready = [&]() __attribute__((always_inline)) {
        if (issued > g + 2) wait_vm<5>();  // raw tile s+2 may still be in flight
        else wait_vm<0>();
      };
      const int tq = ks + kTile * s;  // first key of tile s

      if (has_rows && last) {  // the segment's last step has no QK
        if constexpr (QF8) {
          if (more) issue_q(ld_uniform(segs + 4 * (si + 1)));
          if (do_dma) dma_q8(dt);
        } else if constexpr (RAWW) {
          if (widen_next) {
            raw_ready();
            static_for<9>([&](auto ic) __attribute__((always_inline)) { widen(raw_slot(g + 1), wst, ic); });
          }
          if (more) issue_q(ld_uniform(segs + 4 * (si + 1)));
          if (do_dma) dma_raw(dt);
        } else {
          if (more) issue_q(ld_uniform(segs + 4 * (si + 1)));
          if (do_dma) dma_all(dt);
        }
        dma_last = do_dma;
      }
      if (has_rows) {
        // the DMA goes between the QK MFMAs unless the tile ends inside this wave's rows
        // (then it is issued here, with the clamped offsets)
        const bool dma_il = !FP8 && do_dma && (!FAST || dt.kmax >= wkey);  // wave-uniform
        if (!FP8 && !last && do_dma && !dma_il) dma_all(dt);
        // fp8 (pages of 32 keys): this wave's rows of tile s+1 widened at once, before the
        // QK chain (spread between its MFMAs, the widening's LDS writes stall the K reads
        // longer than the whole widening takes here)
        if (RAWW && !last && widen_next) {
          raw_ready();
          if constexpr (FAST) widen_all(raw_slot(g + 1), wst);
        }
        if (QF8 && !last && do_dma) dma_q8(dt);
        // ---- fp8 queries: S^T = K . Q^T in 9 fp8 k-steps of 64 dims over the raw tile,
        // with this wave's rows of the tile's value columns widened between them ----
        if constexpr (QF8) {
          if (!last) {
            const char* kp8 = smem + qst + kq8base;
            auto k8_at = [&](int c) __attribute__((always_inline)) {
              return cat8(*(const u32x4_t*)(kp8 + 64 * c), *(const u32x4_t*)(kp8 + 64 * c + 16));
            };
            constexpr int KR8 = 3;
            u32x8_t kb8[KR8];
#pragma unroll
            for (int c = 0; c < KR8; ++c) kb8[c] = k8_at(c);
            u32x4_t wr[4];
            widen8_read(qst, wr);
            static_for<9>([&](auto kc) __attribute__((always_inline)) {
              constexpr int c = decltype(kc)::value;
              const u32x8_t qb = cat8(qr[2 * c], qr[2 * c + 1]);
              if constexpr (c == 0)
                mfma8_first(sc, kb8[0], qb);
              else if constexpr (c == 8)
                mfma8_last(sc, kb8[c % KR8], qb);
              else
                mfma8_acc(sc, kb8[c % KR8], qb);
              if constexpr (c + KR8 < 9) kb8[c % KR8] = k8_at(c + KR8);
              if constexpr (c >= 1 && c <= 4) widen8_part(wst, wr, c - 1);
            });
          }
        }
        // ---- S^T[32 keys][32 rows] = K . Q^T: 36 k-steps over the 576 dims, with this
        // wave's DMA of a later tile between the MFMAs ----
        if (!QF8 && !last) {
          const char* kp = smem + qst + kbase;
          auto k_at = [&](int k) __attribute__((always_inline)) { return *(const u32x4_t*)(kp + 32 * k); };
          constexpr int KR = KRING;
          u32x4_t kb[KR];
#pragma unroll
          for (int k = 0; k < KR; ++k) kb[k] = k_at(k);
          // the first DMA steps fill the wait for the first K fragments
          if constexpr (!FP8)
            static_for<DMA0>([&](auto nc) __attribute__((always_inline)) {
              if (dma_il) dma_one(dt, nc);
            });
          static_for<36>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            if constexpr (QF8) {
              // (not reached: the fp8-query chain above)
            } else if constexpr (k == 0)
              mfma_v_first_nw(sc, kb[0], qr[0]);
            else if constexpr (k == 35)
              mfma_acc_v_last(sc, kb[k % KR], qr[k]);
            else
              mfma_acc_v(sc, kb[k % KR], qr[k]);
            if constexpr (k + KR < 36) kb[k % KR] = k_at(k + KR);
            constexpr int n = DMA0 + k / 3;
            if constexpr (!FP8 && k % 3 == 2 && n < 10) {
              if (dma_il) dma_one(dt, std::integral_constant<int, n>{});
            }
            // fp8, generic pages: widen this wave's rows of tile s+1 between the MFMAs
            if constexpr (RAWW && !FAST && k >= 2 && k % 3 == 2 && k / 3 < 9) {
              if (widen_next) widen(raw_slot(g + 1), wst, std::integral_constant<int, k / 3>{});
            }
            // fp8: load raw tile s+3 into the slot the widening freed
            if constexpr (RAWW && k == 30) {
              if (do_dma) dma_raw(dt);
            }
          });
        }

        // ---- softmax of tile s, spread over the P.V chain below (lane: row 32w + r32;
        // element v holds key row_key(8(v/4) + 4 h2 + v%4) of the tile).  The
        // exponentials are taken against the current reference (exponent offset nm); it
        // stands unless a key exceeds it by more than 2^8, which this lane can test on its
        // own maximum against thr (the reference plus 8, in units of S).  When some lane
        // fails the test (a segment's first visible keys, then rarely) the tile is redone
        // after the chain.  Every op is a volatile statement in a fixed slot after an
        // MFMA, at least one slot after the ops it reads. ----
        if (last || tq + kTile > lim_lo) {  // wave-uniform: some key of the tile is masked
          const int rem = last ? 0 : lim - tq;  // tile key k is visible iff k < rem
          // element v holds key h2 + row_key(8(v/4) + v%4): compare with rem - h2 (the lane
          // half recomputed here rather than 16 key indices held across the loop)
          const int remh = rem - (lane_now() >> 5);
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (row_key(8 * (v >> 2) + (v & 3)) >= remh) sc[v] = -INFINITY;
        }
        float mt[5], mf, mg, mx, ar[16], ex[16], tp[8], psum = 0.f, prnd = 0.f;
        uint32_t pk4[4];  // P of pairs 4..7 as bf16, moved into the P.V operand after the chain
        auto slot = [&](auto ic) __attribute__((always_inline)) {
          constexpr int i = decltype(ic)::value;
          // this lane's maximum: a tree of v_max3 over slots 0..3
          if constexpr (i == 0) {
            vmax3(mt[0], sc[0], sc[1], sc[2]);
            vmax3(mt[1], sc[3], sc[4], sc[5]);
            vmax3(mt[2], sc[6], sc[7], sc[8]);
          }
          if constexpr (i == 1) {
            vmax3(mt[3], sc[9], sc[10], sc[11]);
            vmax3(mt[4], sc[12], sc[13], sc[14]);
            vmax3(mf, mt[0], mt[1], mt[2]);
          }
          if constexpr (i == 2) vmax3(mg, mt[3], mt[4], sc[15]);
          if constexpr (i == 3) vmax3(mx, mf, mg, mg);
          // pair k = elements 2k, 2k+1: fma at slot F, exp at F+1, pair sum at F+2, row sum
          // and bf16 pack at F+3; pairs 4..7 first (packed into pk4 until their old P.V
          // operand is dead), then pairs 0..3, packed in place once the first k-step's
          // MFMAs are issued.  The exact row sum (psum) gives the LSE, the sum of the
          // packed values (prnd) normalises the output.
          static_for<8>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            constexpr int F = k >= 4 ? 2 + 2 * (k - 4) : 14 + 2 * k;
            if constexpr (i == F) {
              vfma(ar[2 * k], sc[2 * k], c, nm);
              vfma(ar[2 * k + 1], sc[2 * k + 1], c, nm);
            }
            if constexpr (i == F + 1) {
              vexp2(ex[2 * k], ar[2 * k]);
              vexp2(ex[2 * k + 1], ar[2 * k + 1]);
            }
            if constexpr (i == F + 2) vadd(tp[k], ex[2 * k], ex[2 * k + 1]);
            if constexpr (i == F + 3) {
              vadd(psum, psum, tp[k]);
              if constexpr (k < 4) {
                uint32_t pk;
                vcvt_bf16x2(pk, ex[2 * k], ex[2 * k + 1]);
                pq[0][k] = pk;
              } else {
                vcvt_bf16x2(pk4[k - 4], ex[2 * k], ex[2 * k + 1]);
              }
            }
            if constexpr (i == F + 4) {
              dot2_sum(prnd, k < 4 ? pq[0][k] : pk4[k - 4]);
              use(prnd);
            }
          });
        };

        // ---- O^T[32 cols][32 rows] += V^T . P^T of tile s-1, 16 keys per k-step ----
        // B operand: P^T = elements 8s'..8s'+7 of the previous tile's S^T (as bf16).
        {
          const char* vp = smem + pst + vbase;
          auto vt_at = [&](int i) __attribute__((always_inline)) {  // fragment i = 16 s' + cb
            const char* p = vp + (i >> 4) * 16 * kRowB + 64 * (i & 15);
            return read_vt(p, p + 2 * kRowB);
          };
          constexpr int VR = 3;
          u32x4_t vb[VR];
#pragma unroll
          for (int i = 0; i < VR; ++i) vb[i] = vt_at(i);
          const u32x4_t p0 = pq[0], p1 = pq[1];
          static_for<32>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            constexpr int sk = i >> 4, cb = i & 15;
            mfma_a_nw(O[cb], vb[i % VR], sk ? p1 : p0);
            if constexpr (i + VR < 32) vb[i % VR] = vt_at(i + VR);
            slot(ic);
          });
        }

        float fac = 1.f;
        if (__any(mx > thr)) {
          // redo the tile against a raised reference: the row maximum (both halves), the
          // factor for O and l (1 for the segment's first visible keys), new exponentials
          const float mr = half_max(mx) * c;
          const float m_new = fmaxf(m_ref, mr);
          fac = (m_new > m_ref && m_ref != -INFINITY) ? fast_exp2(m_ref - m_new) : 1.f;
          m_ref = m_new;
          nm = (m_ref == -INFINITY) ? 0.f : -m_ref;  // exp2(-inf) = 0 covers masked keys
          thr = (m_ref == -INFINITY) ? -INFINITY : (m_ref + kRescaleAt) / c;
          float ps = 0.f, pr = 0.f;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float e0 = fast_exp2(fmaf(sc[2 * k], c, nm)), e1 = fast_exp2(fmaf(sc[2 * k + 1], c, nm));
            const uint32_t pk = pack_bf16x2(e0, e1);
            ps += e0 + e1;
            dot2_sum(pr, pk);
            pq[k >> 2][k & 3] = pk;
          }
          l_acc = l_acc * fac + ps;
          l_rnd = l_rnd * fac + pr;
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) pq[1][k] = pk4[k];
          l_acc += psum;
          l_rnd += prnd;
        }
        // rare: O holds P.V up to tile s-1, taken against the old reference
        if (__any(fac != 1.f)) {
          asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");  // the last P.V MFMA's result
#pragma unroll
          for (int cb = 0; cb < 16; ++cb) {
            acc_fence(O[cb]);
#pragma unroll
            for (int v = 0; v < 16; ++v) O[cb][v] *= fac;
            acc_written(O[cb]);
          }
        }
      } else {
        if constexpr (QF8) {
          // no query rows: only this wave's share of the DMA and of the widening
          if (!last) {
            u32x4_t wr[4];
            widen8_read(qst, wr);
#pragma unroll
            for (int i = 0; i < 4; ++i) widen8_part(wst, wr, i);
          }
          if (do_dma) dma_q8(dt);
        } else if constexpr (RAWW) {
          if (widen_next) {
            raw_ready();
            static_for<9>([&](auto ic) __attribute__((always_inline)) { widen(raw_slot(g + 1), wst, ic); });
          }
          if (do_dma) dma_raw(dt);
        } else {
          if (do_dma) dma_all(dt);
        }
      }
      if (do_dma) {
        pf = next_tile(segs, pf, s_end);
        issued++;
      }
      if (widen_next) widened++;
    }
    done = g0 + nt;
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");  // the last P.V MFMA's result is read next
    // the next segment's queries (issued in the last step, or here after an empty segment)
    if (has_rows && more) {
      if (nt == 0) {
        issue_q(ld_uniform(segs + 4 * (si + 1)));
        wait_vm<0>();
      } else if (!dma_last) {
        wait_vm<0>();
      } else if constexpr (QF8) {
        if (w == 3) wait_vm<4>();
        else wait_vm<5>();
      } else if constexpr (RAWW) {
        wait_vm<5>();
      } else {
        if (w0) wait_vm<10>();
        else wait_vm<9>();
      }
      q_landed();
    }

    // ---- epilogue: o = O * kv_scale / l, lse = ln(sum exp) ----
    if (has_rows) {
      const float l_row = half_sum(l_acc);  // exact row sum: the LSE
      const float l_out = half_sum(l_rnd);  // sum of the rounded probabilities: normalises O
      // split rows: the partial is stored as fp16 O * psc, psc a power of two that puts
      // the row's largest |O| in [2^14, 2^15) (the row sum is stored with the same factor)
      float psc = 1.f;
      if (pidx >= 0) {
        float am = 0.f;
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) {
          acc_fence(O[cb]);
#pragma unroll
          for (int v = 0; v < 16; ++v) am = fmaxf(am, fabsf(O[cb][v]));
        }
        am = half_max(am);
        const int E = am > 0.f ? __builtin_amdgcn_frexp_expf(am) : 15;
        psc = __builtin_ldexpf(1.f, min(max(15 - E, -64), 64));
      }
      const int ln = lane_now(), hl = ln >> 5;
      const int rl = 32 * w + (ln & 31);
      if (rl < RG) {
        const int r = row0 + rl;
        const float lse = (l_row > 0.f) ? (m_ref + fast_log2(l_row)) * kLn2 : -INFINITY;
        const float f = (l_out > 0.f) ? a.out_scale / l_out : 0.f;
        int t, h;
        row_th(ln & 31, t, h);
        if (pidx < 0) {
          if (a.lse && hl == 0) a.lse[((int64_t)b * a.Sq + t) * a.N + h] = lse;
          uint16_t* orow = a.o + ((int64_t)b * a.Sq + t) * a.o_s_tok + (int64_t)h * a.o_s_head;
#pragma unroll
          for (int cb = 0; cb < 16; ++cb) {
            acc_fence(O[cb]);
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int col = 32 * cb + 8 * gq + 4 * hl;
              u32x2_t pk2;
              pk2[0] = pack_bf16x2(O[cb][4 * gq] * f, O[cb][4 * gq + 1] * f);
              pk2[1] = pack_bf16x2(O[cb][4 * gq + 2] * f, O[cb][4 * gq + 3] * f);
              *(u32x2_t*)(orow + col) = pk2;
            }
          }
        } else {
          if (hl == 0) {
            a.ws_lse[(int64_t)pidx * R + r] = lse;
            a.ws_l[(int64_t)pidx * R + r] = l_out / a.out_scale * psc;
          }
          // unnormalised, scaled partial block of rows row0 + 32w .. +31 as fp16 (the reduce
          // divides by the stored row sums) in accumulator order: chunk pair
          // q = 2 cb + gp holds 64 lanes x 8 values (elements 8 gp .. 8 gp + 7 of O[cb]),
          // so each store is 1 KB contiguous
          char* pblk = (char*)a.ws_o + ((int64_t)pidx * partial_rows(a.Sq, a.N) + row0 + 32 * w) * kLkv * 2;
#pragma unroll
          for (int cb = 0; cb < 16; ++cb) {
            acc_fence(O[cb]);
#pragma unroll
            for (int gp = 0; gp < 2; ++gp)
              *(u32x4_t*)(pblk + 16 * (64 * (2 * cb + gp) + ln)) =
                  u32x4_t{pack_f16x2(O[cb][8 * gp] * psc, O[cb][8 * gp + 1] * psc),
                          pack_f16x2(O[cb][8 * gp + 2] * psc, O[cb][8 * gp + 3] * psc),
                          pack_f16x2(O[cb][8 * gp + 4] * psc, O[cb][8 * gp + 5] * psc),
                          pack_f16x2(O[cb][8 * gp + 6] * psc, O[cb][8 * gp + 7] * psc)};
          }
        }
      }
    }
  }
  wait_vm<0>();  // no DMA outlives the workgroup
}

hipError_t launch_decode(const DecodeArgs& a, bool fp8, bool qf8, hipStream_t stream) {
  const int parts8 = (a.num_parts + 7) / 8 * 8;
  const dim3 grid(parts8 * a.head_groups);
  const bool p32 = (a.page_size % 32) == 0;
  if (fp8) {
    const bool canon = (const char*)a.k_pe == (const char*)a.kv_c + kLkv;
    if (qf8) {
      if (p32 && canon) hipLaunchKernelGGL((mla_decode_pipe_kernel<true, true, true>), grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL((mla_decode_pipe_kernel<false, true, true>), grid, dim3(256), 0, stream, a);
    } else {
      if (p32 && canon) hipLaunchKernelGGL((mla_decode_pipe_kernel<true, true, false>), grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL((mla_decode_pipe_kernel<false, true, false>), grid, dim3(256), 0, stream, a);
    }
  } else {
    // one base for the whole cache row: the rope columns follow the latent ones
    const bool canon = (const char*)a.k_pe == (const char*)a.kv_c + 2 * kLkv;
    if (p32 && canon) hipLaunchKernelGGL((mla_decode_pipe_kernel<true, false, false>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((mla_decode_pipe_kernel<false, false, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
