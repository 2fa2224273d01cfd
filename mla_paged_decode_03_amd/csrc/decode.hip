// Paged latent-MQA decode kernel for gfx950.
//
// Computes, for every query row of every request, softmax attention over the
// request's cache rows [kv_c | k_pe] with value kv_c (vLLM mla/common.py
// module docstring, "Data-Movement Friendly Approach").  One workgroup of four
// waves owns one head group (up to 64 query rows of one request) of one plan
// part and walks the part's segments (request, key range) in 32-key tiles.
// The head groups of a part run on one XCD, so a tile read from HBM by one of
// them is served to the others from that XCD's L2.
//
//  load     a tile is 32 cache rows of 576 bf16 (36 KB) in LDS: a latent part
//           [32 rows][512] (1 KB per row) and a rope part [32 rows][64], both
//           row-major with a 16-byte-chunk XOR swizzle.  bf16 caches go HBM ->
//           LDS with global_load_lds_dwordx4 (no VGPRs), one instruction per
//           latent row, so the row address is wave-uniform; up to 3 tiles are
//           in flight ahead of the one being computed.  fp8 caches go through
//           VGPRs, are widened to bf16 and written to LDS.  Keys past the
//           segment end load a valid key instead and get probability 0, so
//           unused page slots and block_table entries are never read.
//  QK^T     wave w < ceil(rows/32) computes S^T[32 keys x 32 rows] for rows
//           32w..32w+31 with v_mfma_f32_32x32x16_bf16: A = K rows from LDS,
//           B = the wave's query rows, held in VGPRs for the whole segment.
//  softmax  fp32, log2 domain; row max / sum over the two lane halves of the
//           MFMA layout.  Each row's reference max is fixed by its first tile
//           with a visible key and O is never rescaled: if a later tile exceeds
//           the reference by more than 2^64 the workgroup restarts the segment
//           with the raised maxima (a bounded number of times), so P <= 2^64
//           and O stays in AGPRs as a plain MFMA accumulator.  P (bf16) -> LDS.
//  P.V      wave w owns output columns 128w..128w+127 of every row and
//           accumulates O^T += V^T . P^T.  V^T fragments come straight from the
//           row-major K tile through ds_read_b64_tr_b16 (4 keys x 16 columns
//           per 16-lane group), P fragments from LDS.
//  epilogue o = O * kv_scale / l, lse = ln(sum exp) to the output, or fp32
//           partial states to the workspace when the request is split.
#include "common.h"
#include "kernels.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace mla {

namespace {

constexpr int kTile = 32;
constexpr int kLatRow = kLkv * 2;                 // 1024: latent part of a bf16 key row
constexpr int kRopeRow = kRope * 2;               // 128: rope part
constexpr int kRopeOff = kTile * kLatRow;         // 32768: rope part of a stage
constexpr int kStageBytes = kRopeOff + kTile * kRopeRow;  // 36864
constexpr int kMaxStages = 4;
constexpr int kPOff = kMaxStages * kStageBytes;   // 147456: P [128 rows][4 chunks][8 keys] bf16
constexpr int kEllOff = kPOff + 128 * 64;         // 155648: row sums for the epilogue
constexpr int kFlagOff = kEllOff + 128 * 4;       // 156160: per-wave restart request
constexpr int kSmemBytes = kFlagOff + 16;         // 156176
constexpr float kMaxOvershoot = 64.f;             // log2 units

__shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// Keeps an MFMA accumulator in AGPRs.  The constraint also makes the compiler select
// the AGPR form of every MFMA in the kernel, so accumulators that only MFMAs update
// stay in the accumulation registers instead of being copied to VGPRs and back.
template <typename T>
__device__ __forceinline__ void pin_agpr(T& x) { asm("" : "+a"(x)); }

// The lane index, produced by a volatile instruction pair so that per-lane values
// derived from it are recomputed where they are used instead of being hoisted out
// of the loops and kept live (VGPRs are the scarce resource of this kernel).
__device__ __forceinline__ int lane_id() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// HBM -> LDS, 16 bytes per lane: lane l writes LDS bytes [m0 + 16 l, m0 + 16 l + 16).
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}
// Waits until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// A tile is PER DMA instructions per wave; wait until at most `newer` tiles are pending.
template <int PER>
__device__ __forceinline__ void wait_tiles(int newer) {
  switch (newer) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<PER>(); break;
    default: wait_vm<2 * PER>(); break;
  }
}
// Same, with a uniform 64-bit global base and a 32-bit per-lane offset.
__device__ __forceinline__ void dma16_s(const void* gbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds_base)
               : "memory", "m0");
}
// Workgroup barrier that also orders this wave's LDS writes (and does not drain vmcnt).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS swizzles (64 banks of 4 bytes: a 16-byte chunk's bank group is its index mod 16).
// Latent rows are 1 KB apart, so every row starts in the same bank group; logical chunk
// c of key k sits in physical chunk c ^ lat_swz(k).  lat_swz is a bijection on k & 15,
// so the 16 keys of one ds_read_b128 cycle (same c) hit 16 distinct bank groups, and for
// any 4 consecutive keys 4a..4a+3 it gives 4 distinct chunk pairs, so the transposing
// V reads (4 keys x 2 chunks per 16-lane group) are conflict-free too.
__device__ __forceinline__ int lat_swz(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }
// Rope rows are 128 B (8 chunks): keys 2m and 2m+1 share bank groups 0..7 / 8..15, so
// the keys of one parity need distinct chunks.
__device__ __forceinline__ int rope_swz(int k) { return (k >> 1) & 7; }

// Byte offset in a stage of logical 16-byte chunk c (0..71) of key row `key`: the
// latent row (c < 64) or the rope row (c >= 64), swizzled as above.
__device__ __forceinline__ int tile_off(int key, int c) {
  return c < 64 ? key * kLatRow + ((c ^ lat_swz(key)) << 4)
                : kRopeOff + key * kRopeRow + (((c - 64) ^ rope_swz(key)) << 4);
}

__device__ __forceinline__ int p_off(int row, int q) {  // P tile [row][chunk q of 8 keys]
  return row * 64 + ((q ^ ((row >> 1) & 3)) << 4);
}

struct Seg {
  int b, ks, ke, pidx;
};
__device__ __forceinline__ Seg load_seg(const int32_t* segs, int si) {
  return Seg{ld_uniform(segs + 4 * si), ld_uniform(segs + 4 * si + 1), ld_uniform(segs + 4 * si + 2),
             ld_uniform(segs + 4 * si + 3)};
}

// Tile cursor over the part's segments: (segment index, first key of the tile).
struct Cursor {
  int si, ts;
};
__device__ __forceinline__ Cursor first_tile(const int32_t* segs, int si, int s_end) {
  for (; si < s_end; ++si) {
    const Seg s = load_seg(segs, si);
    if (s.ke > s.ks) return Cursor{si, s.ks};
  }
  return Cursor{s_end, 0};
}
__device__ __forceinline__ Cursor next_tile(const int32_t* segs, Cursor c, int s_end) {
  const Seg s = load_seg(segs, c.si);
  if (c.ts + kTile < s.ke) return Cursor{c.si, c.ts + kTile};
  return first_tile(segs, c.si + 1, s_end);
}

// Byte offset (from the cache base) of key row j of a request; esz = element size.
// UNIFORM: j is the same in every lane (scalar block_table load).
template <bool UNIFORM>
__device__ __forceinline__ int64_t row_bytes(const DecodeArgs& a, const int32_t* bt_row, int j, int esz) {
  const unsigned ps = (unsigned)a.page_size;
  const int page = UNIFORM ? ld_uniform(bt_row + (unsigned)j / ps) : bt_row[(unsigned)j / ps];
  return ((int64_t)page * a.s_page + (int64_t)((unsigned)j % ps) * a.s_tok) * esz;
}

// bf16: issue this wave's DMA loads of tile (b, keys ts..ts+31 clipped at ke) into
// `stage`: wave w loads key rows 8w..8w+7, one instruction per latent row (lane =
// physical chunk) and the rope parts of its 8 rows (lane = 8 rows x 8 chunks).  A key
// past ke loads key ke-1 instead.  Returns nothing; PER_TILE instructions per wave.
template <bool PAGED32>
__device__ __forceinline__ void issue_tile_bf16(const DecodeArgs& a, int b, int ts, int ke, uint32_t stage,
                                                int w, int lane) {
  const int32_t* bt_row = a.block_table + (int64_t)b * a.bt_s;
  const char* kvc = (const char*)a.kv_c;
  const char* kpe = (const char*)a.k_pe;
  const int kmax = ke - ts - 1;
  const int64_t s_tok2 = a.s_tok * 2;
  int64_t tile_base = 0;
  if constexpr (PAGED32) tile_base = row_bytes<true>(a, bt_row, ts, 2);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int key = 8 * w + i;  // wave-uniform
    const int kc = min(key, kmax);
    const int64_t roff = PAGED32 ? tile_base + kc * s_tok2 : row_bytes<true>(a, bt_row, ts + kc, 2);
    dma16_s(kvc + roff, (uint32_t)((lane ^ lat_swz(key)) << 4),
            __builtin_amdgcn_readfirstlane(stage + key * kLatRow));
  }
  // rope: lane = (row 8w + lane/8, physical chunk lane%8)
  const int rk = 8 * w + (lane >> 3);
  const uint32_t rlds = __builtin_amdgcn_readfirstlane(stage + kRopeOff + 8 * w * kRopeRow);
  if constexpr (PAGED32) {
    const int kc = min(rk, kmax);
    const uint32_t voff = (uint32_t)(kc * s_tok2) + ((((lane & 7) ^ rope_swz(rk))) << 4);
    dma16_s(kpe + tile_base, voff, rlds);
  } else {
    // rows may sit on different pages: one instruction per row with only its 8 lanes active
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = 8 * w + i;
      const int kc = min(key, kmax);
      const int64_t roff = row_bytes<true>(a, bt_row, ts + kc, 2);
      if ((lane >> 3) == i) dma16_s(kpe + roff, (uint32_t)((((lane & 7) ^ rope_swz(key))) << 4), rlds);
    }
  }
}

// fp8: per thread 9 chunks of 8 bytes (8 dims); chunk u = tid + 256 i of the tile.
template <bool PAGED32>
__device__ __forceinline__ void load_tile_fp8(const DecodeArgs& a, int b, int ts, int ke, int tid,
                                              u32x2_t (&v)[9]) {
  const int32_t* bt_row = a.block_table + (int64_t)b * a.bt_s;
  const char* kvc = (const char*)a.kv_c;
  const int64_t pe_delta = (const char*)a.k_pe - kvc;
  const int kmax = ke - ts - 1;
  int64_t tile_base = 0;
  if constexpr (PAGED32) tile_base = row_bytes<true>(a, bt_row, ts, 1);
  int64_t off[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int u = tid + 256 * i;
    const int kk = min(u / 72, kmax), c = u - 72 * (u / 72);
    const int64_t o = PAGED32 ? tile_base + (int64_t)kk * a.s_tok : row_bytes<false>(a, bt_row, ts + kk, 1);
    off[i] = o + ((c < 64) ? (int64_t)(8 * c) : pe_delta + 8 * (c - 64));
  }
#pragma unroll
  for (int i = 0; i < 9; ++i) v[i] = *(const u32x2_t*)(kvc + off[i]);
}

__device__ __forceinline__ void store_tile_fp8(char* stage, int tid, const u32x2_t (&v)[9]) {
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int u = tid + 256 * i;
    const int kk = u / 72, c = u - 72 * (u / 72);
    const u32x2_t lo = fp8x4_to_bf16x4(v[i][0]);
    const u32x2_t hi = fp8x4_to_bf16x4(v[i][1]);
    *(u32x4_t*)(stage + tile_off(kk, c)) = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  }
}

// 8 bf16 of V^T (column of this lane, 8 keys) from the row-major tile: two transposing
// reads, p0 for keys t0..t0+3 and p1 for keys t0+8..t0+11.
__device__ __forceinline__ u32x4_t read_vt(const char* p0, const char* p1) {
  const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const lds_char*)p0);
  const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const lds_char*)p1);
  u32x4_t r;
  r[0] = (uint32_t)(uint16_t)v0[0] | ((uint32_t)(uint16_t)v0[1] << 16);
  r[1] = (uint32_t)(uint16_t)v0[2] | ((uint32_t)(uint16_t)v0[3] << 16);
  r[2] = (uint32_t)(uint16_t)v1[0] | ((uint32_t)(uint16_t)v1[1] << 16);
  r[3] = (uint32_t)(uint16_t)v1[2] | ((uint32_t)(uint16_t)v1[3] << 16);
  return r;
}

// Issues up to `count` tiles at the cursor: DMA into the next stages (bf16) or the
// staging registers (fp8).
template <bool FP8, bool PAGED32, int NST>
__device__ __forceinline__ void issue_ahead(const DecodeArgs& a, const int32_t* segs, int s_end,
                                            Cursor& pf, int& issued, int count, int tid, int w, int l,
                                            u32x2_t (&fstage)[9]) {
  for (int k = 0; k < count; ++k) {
    if (pf.si >= s_end) break;
    const Seg s = load_seg(segs, pf.si);
    if constexpr (FP8)
      load_tile_fp8<PAGED32>(a, s.b, pf.ts, s.ke, 64 * w + lane_id(), fstage);
    else
      issue_tile_bf16<PAGED32>(a, s.b, pf.ts, s.ke, lds_addr(smem) + (issued % NST) * kStageBytes, w,
                               lane_id());
    pf = next_tile(segs, pf, s_end);
    issued++;
  }
}

}  // namespace

template <bool FP8, bool PAGED32, int NRB>
__global__ __launch_bounds__(256, 1) void mla_decode_kernel(DecodeArgs a) {
  constexpr int NST = FP8 ? 2 : kMaxStages;
  const int tid = threadIdx.x, l = tid & 63, l32 = l & 31, hh = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in an SGPR

  // Workgroups are dealt round-robin to the 8 XCDs; keep the head groups of
  // one part on one XCD so that they share its L2 for the part's keys.
  const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const int hg = slot % a.head_groups;
  const int part = xcd + 8 * (slot / a.head_groups);
  if (part >= a.num_parts) return;

  const int R = a.Sq * a.N;
  const int row0 = hg * kGroupRows;
  const int RG = min(kGroupRows, R - row0);  // rows of this group; NRB = ceil(RG / 32) or more
  const int32_t* segs = a.segs;
  const int s_beg = ld_uniform(a.part_begin + part), s_end = ld_uniform(a.part_begin + part + 1);

  float* ell_l = (float*)(smem + kEllOff);
  int* flag_l = (int*)(smem + kFlagOff);

  const int qrow_loc = 32 * w + l32;  // this lane's query row in QK^T (waves w < NRB)
  const bool qk_wave = w < NRB;

  // ---- load pipeline (wave-uniform state) ----
  Cursor pf = first_tile(segs, s_beg, s_end);  // next tile to load
  int issued = 0, consumed = 0;
  u32x2_t fstage[9];  // fp8 staging registers

  issue_ahead<FP8, PAGED32, NST>(a, segs, s_end, pf, issued, NST - 1, tid, w, l, fstage);

  for (int si = s_beg; si < s_end; ++si) {
    const Seg sg = load_seg(segs, si);
    const int b = sg.b, ks = sg.ks, ke = sg.ke, pidx = sg.pidx;
    const int L = ld_uniform(a.seq_lens + b);

    // Query rows of this wave: B operand of S^T = K . Q^T, 36 x 8 bf16 per lane.
    u32x4_t qr[36];
    int lim = 0;  // keys j < lim are visible to this row (segment end, causal window)
    if (qk_wave) {
      const int r = row0 + qrow_loc;
      if (qrow_loc < RG) {
        const int t = r / a.N, h = r - t * a.N;
        const int64_t tok = (int64_t)b * a.Sq + t;
        const uint16_t* qn = a.q_nope + tok * a.q_nope_s_tok + (int64_t)h * a.q_nope_s_head + 8 * hh;
        const uint16_t* qp = a.q_pe + tok * a.q_pe_s_tok + (int64_t)h * a.q_pe_s_head + 8 * hh;
#pragma unroll
        for (int k = 0; k < 32; ++k) qr[k] = *(const u32x4_t*)(qn + 16 * k);
#pragma unroll
        for (int k = 0; k < 4; ++k) qr[32 + k] = *(const u32x4_t*)(qp + 16 * k);
        // A wait the compiler sees: the query loads are complete before the tile loop,
        // so it places no vmcnt waits there (they would also count the DMA loads in
        // flight and drain the prefetch pipeline).  s_waitcnt vmcnt(0).
        __builtin_amdgcn_s_waitcnt(0x0F70);
        lim = min(ke, L - (a.Sq - 1) + t);
      } else {
        // padding rows: zero queries give zero logits; their probabilities only reach
        // output rows that are never stored
#pragma unroll
        for (int k = 0; k < 36; ++k) qr[k] = u32x4_t{0, 0, 0, 0};
        lim = ke;
      }
    }

    float m_ref = -INFINITY;   // reference max of this row (log2 units)
    float m_seen = -INFINITY;  // largest logit seen so far
    float l_run = 0.f;
    f32x16_t O[4][NRB];
    for (;;) {  // one pass over the segment; repeated only after a restart request
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NRB; ++j) {
#pragma unroll
          for (int v = 0; v < 16; ++v) O[i][j][v] = 0.f;
          pin_agpr(O[i][j]);
        }
      l_run = 0.f;
      bool restart = false;

      for (int ts = ks; ts < ke; ts += kTile) {
        char* stage = smem + (consumed % NST) * kStageBytes;
        if constexpr (FP8) {
          // the stage was last read two tiles ago, before the previous barriers
          store_tile_fp8(stage, 64 * w + lane_id(), fstage);
          issue_ahead<FP8, PAGED32, NST>(a, segs, s_end, pf, issued, 1, tid, w, l, fstage);
          barrier_lds();
        } else {
          wait_tiles<PAGED32 ? 9 : 16>(issued - consumed - 1);  // this tile's DMA has landed
          barrier_lds();                      // ... for every wave; the previous stage is free
          issue_ahead<FP8, PAGED32, NST>(a, segs, s_end, pf, issued, 1, tid, w, l, fstage);
        }

        if (qk_wave) {
          // QK A operand: key r32, logical chunk 2k + h2 at byte kq_off[k & 7] + 256 (k >> 3)
          // (latent, k < 32; the swizzle only permutes chunks within a 16-chunk group) or
          // kr_off[k & 3] (rope, k >= 32).
          const int ln = lane_id(), r32 = ln & 31, h2 = ln >> 5;
          int kq_off[8], kr_off[4];
#pragma unroll
          for (int m = 0; m < 8; ++m) kq_off[m] = r32 * kLatRow + (((2 * m + h2) ^ lat_swz(r32)) << 4);
#pragma unroll
          for (int m = 0; m < 4; ++m)
            kr_off[m] = kRopeOff + r32 * kRopeRow + (((2 * m + h2) ^ rope_swz(r32)) << 4);
          // 36 MFMAs over the 576 dims; K fragments stream through a 4-deep ring so that
          // LDS latency overlaps the MFMA chain.
          auto kaddr = [&](int k) -> const u32x4_t* {
            return (const u32x4_t*)(stage + (k < 32 ? kq_off[k & 7] + 256 * (k >> 3) : kr_off[k & 3]));
          };
          u32x4_t kb[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) kb[k] = *kaddr(k);
          f32x16_t sacc;
#pragma unroll
          for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
          for (int k = 0; k < 36; ++k) {
            const u32x4_t kf = kb[k & 3];
            if (k + 4 < 36) kb[k & 3] = *kaddr(k + 4);
            sacc = mfma32(kf, qr[k], sacc);
          }
          // Logits in log2 units are c * s (c = scale * log2 e > 0); masked keys get -inf.
          // Tiles entirely inside every row's window skip the masking.
          const float c = a.qk_scale_log2;
          if (!__all(ts + kTile <= lim)) {
            const int rem = lim - ts - 4 * h2;  // key 8(v/4) + 4 h2 + v%4 is visible iff < lim - ts
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (8 * (v >> 2) + (v & 3) >= rem) sacc[v] = -INFINITY;
          }
          float mx = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[v]);
          mx = half_max(mx) * c;
          m_seen = fmaxf(m_seen, mx);
          if (m_ref == -INFINITY) m_ref = mx;  // first visible keys: O and l are still 0
          const bool over = mx > m_ref + kMaxOvershoot;
          const bool dead = (m_ref == -INFINITY);
          float psum = 0.f;
          uint32_t pk[8];
          const float nm = dead ? 0.f : -m_ref;
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            // exp2(-inf) = 0 covers masked keys and rows without visible keys (c * s = -inf)
            const float p0 = fast_exp2(fmaf(sacc[v], c, nm));
            const float p1 = fast_exp2(fmaf(sacc[v + 1], c, nm));
            psum += p0 + p1;
            pk[v >> 1] = pack_bf16x2(p0, p1);
          }
          psum = half_sum(psum);
          l_run += psum;
          // keys 8s'..8s'+7 of this lane's accumulator form P chunk q = 2s' + h2
          *(u32x4_t*)(smem + kPOff + p_off(32 * w + r32, h2)) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
          *(u32x4_t*)(smem + kPOff + p_off(32 * w + r32, 2 + h2)) = u32x4_t{pk[4], pk[5], pk[6], pk[7]};
          const bool any = __any(over);
          if (l == 0) flag_l[w] = any ? 1 : 0;
        }
        barrier_lds();

#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) restart |= (flag_l[rb] != 0);
        if (restart) break;  // uniform over the workgroup

        // O^T[cols of wave w][rows] += V^T . P^T, 16 keys (one MFMA k-step) at a time.
        // V^T through ds_read_b64_tr_b16: 16-lane group g = lane/16 covers columns
        // c0 = 128w + 32cb + 16(g&1) and keys t0..t0+3, t0 = 16s + 4h (+8 for elements
        // 4..7); lane j = lane%16 addresses key t0 + j/4, columns c0 + 4(j&3) .. +3 and
        // receives keys t0..t0+3 of column c0 + j.
        const int pl = lane_id(), p32 = pl & 31, ph = pl >> 5;
        int vt_off[2][4];  // [key half (+0 / +8)][column block]
        {
          const int g = pl >> 4, j = pl & 15;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            const int key = 4 * ph + (j >> 2) + 8 * kh;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
              const int col = 128 * w + 32 * cb + 16 * (g & 1) + 4 * (j & 3);
              vt_off[kh][cb] = key * kLatRow + (((col >> 3) ^ lat_swz(key)) << 4) + 8 * ((col >> 2) & 1);
            }
          }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          u32x4_t pfr[NRB], vfr[4];
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            pfr[rb] = *(const u32x4_t*)(smem + kPOff + p_off(32 * rb + p32, 2 * s + ph));
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            vfr[cb] = read_vt(stage + vt_off[0][cb] + 16 * s * kLatRow, stage + vt_off[1][cb] + 16 * s * kLatRow);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
              O[cb][rb] = mfma32(vfr[cb], pfr[rb], O[cb][rb]);
              pin_agpr(O[cb][rb]);
            }
        }
        consumed++;
      }
      if (!restart) break;
      // Raise every row's reference to the largest logit seen and start the segment
      // over: drain the loads in flight and refill the pipeline from its first tile.
      m_ref = m_seen;
      wait_vm<0>();
      barrier_lds();
      consumed = issued;
      pf = first_tile(segs, si, s_end);
      issue_ahead<FP8, PAGED32, NST>(a, segs, s_end, pf, issued, NST - 1, tid, w, l, fstage);
    }

    // Epilogue.  QK waves publish the row sums and write the LSE.
    if (qk_wave && hh == 0) {
      ell_l[qrow_loc] = l_run;
      if (qrow_loc < RG) {
        const int r = row0 + qrow_loc;
        const float lse = (l_run > 0.f) ? (m_ref + fast_log2(l_run)) * kLn2 : -INFINITY;
        if (pidx < 0) {
          if (a.lse) {
            const int t = r / a.N, h = r - t * a.N;
            a.lse[((int64_t)b * a.Sq + t) * a.N + h] = lse;
          }
        } else {
          a.ws_lse[(int64_t)pidx * R + r] = lse;
        }
      }
    }
    barrier_lds();
    const int el = lane_id(), e32 = el & 31, eh = el >> 5;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int rl = 32 * rb + e32;
      if (rl >= RG) continue;
      const int r = row0 + rl;
      const float lsum = ell_l[rl];
      const float f = (lsum > 0.f) ? a.out_scale / lsum : 0.f;
      if (pidx < 0) {
        const int t = r / a.N, h = r - t * a.N;
        uint16_t* orow = a.o + ((int64_t)b * a.Sq + t) * a.o_s_tok + (int64_t)h * a.o_s_head;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = 128 * w + 32 * cb + 8 * g + 4 * eh;
            const f32x16_t& acc = O[cb][rb];
            u32x2_t pk;
            pk[0] = pack_bf16x2(acc[4 * g] * f, acc[4 * g + 1] * f);
            pk[1] = pack_bf16x2(acc[4 * g + 2] * f, acc[4 * g + 3] * f);
            *(u32x2_t*)(orow + col) = pk;
          }
      } else {
        float* prow = a.ws_o + ((int64_t)pidx * R + r) * kLkv;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = 128 * w + 32 * cb + 8 * g + 4 * eh;
            const f32x16_t& acc = O[cb][rb];
            *(f32x4_t*)(prow + col) =
                f32x4_t{acc[4 * g] * f, acc[4 * g + 1] * f, acc[4 * g + 2] * f, acc[4 * g + 3] * f};
          }
      }
    }
  }
  wait_vm<0>();  // no DMA outlives the workgroup
}

template <bool FP8, bool PAGED32>
static hipError_t launch_nrb(const DecodeArgs& a, int nrb, dim3 grid, hipStream_t stream) {
  switch (nrb) {
    case 1: hipLaunchKernelGGL((mla_decode_kernel<FP8, PAGED32, 1>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((mla_decode_kernel<FP8, PAGED32, 2>), grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, bool fp8, hipStream_t stream) {
  // Every head group but the last has 64 rows; the last may be smaller, but a
  // group never needs more row blocks than the first one, so one instance serves all.
  const int R = a.Sq * a.N;
  const int nrb = (min(R, kGroupRows) + 31) / 32;
  const int parts8 = (a.num_parts + 7) / 8 * 8;
  const dim3 grid(parts8 * a.head_groups);
  const bool p32 = (a.page_size % 32) == 0;
  if (fp8)
    return p32 ? launch_nrb<true, true>(a, nrb, grid, stream) : launch_nrb<true, false>(a, nrb, grid, stream);
  return p32 ? launch_nrb<false, true>(a, nrb, grid, stream) : launch_nrb<false, false>(a, nrb, grid, stream);
}

}  // namespace mla
