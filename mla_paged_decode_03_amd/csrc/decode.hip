// Paged latent-MQA decode kernel for gfx950.
//
// Computes, for every query row of every request, softmax attention over the
// request's cache rows [kv_c | k_pe] with value kv_c (vLLM mla/common.py
// module docstring, "Data-Movement Friendly Approach").  One workgroup of four
// waves owns one head group (up to 128 query rows of one request) of one plan
// part and walks the part's segments (request, key range) in 32-key tiles:
//
//  stage    every thread loads 16-byte pieces of 8 keys (and one rope piece)
//           from HBM, writes them row-major into the K tile in LDS and, after
//           an 8x8 transpose in registers, key-packed into the V^T tile (the
//           first 512 columns of the same rows are the values).  The loads for
//           the next tile are issued before this tile is consumed.
//  QK^T     wave w < ceil(rows/32) computes S^T[32 keys x 32 rows] for rows
//           32w..32w+31 with v_mfma_f32_32x32x16_bf16: A = K tile (LDS),
//           B = the wave's query rows, held in VGPRs for the whole segment.
//  softmax  online, fp32, log2 domain; row max / sum over the two lane halves
//           of the MFMA layout.  P (bf16) goes to LDS.  Each row's reference
//           max is fixed by its first tile with a visible key and O is never
//           rescaled: if a later tile exceeds the reference by more than
//           2^64, the workgroup restarts the segment with the raised maxima
//           (a bounded number of times), so P <= 2^64 and O stays in AGPRs
//           as a plain MFMA accumulator.
//  P.V      wave w owns output columns 128w..128w+127 of every row and
//           accumulates O^T += V^T . P^T (A = V^T tile, B = P), fp32 in VGPRs.
//  epilogue o = O * kv_scale / l, lse = ln(sum exp) to the output, or fp32
//           partial states to the workspace when the request is split.
//
// Keys at or past the segment end are never loaded (zeros go to LDS) and get
// probability 0, so unused page slots and block_table entries are never read.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kTile = 32;
constexpr int kKRowBytes = kHead * 2;                 // 1152: one bf16 key row
constexpr int kKStageBytes = kTile * kKRowBytes;      // 36864
constexpr int kVtStageBytes = 4 * kLkv * 16;          // 32768: [4 key chunks][512 cols][8 keys]
constexpr int kKOff = 0;
constexpr int kVtOff = 2 * kKStageBytes;              // 73728
constexpr int kPOff = kVtOff + 2 * kVtStageBytes;     // 139264: [128 rows][4 chunks][8 keys] bf16
constexpr int kEllOff = kPOff + 128 * 64;             // 147456: row sums for the epilogue
constexpr int kFlagOff = kEllOff + 128 * 4;           // 147968: per-wave restart request
constexpr int kSmemBytes = kFlagOff + 16;             // 147984
// A logit may exceed its row's reference max by at most this (log2 units)
// before the segment is restarted with a higher reference.
constexpr float kMaxOvershoot = 64.f;

// Key (0..31 within the tile) held at element e of 8-key chunk q of the V^T and
// P layouts.  The order matches where a lane of the 32x32 S^T accumulator
// finds its keys, so P needs no shuffle between the two MFMAs.
__device__ __forceinline__ int chunk_key(int q, int e) {
  return 16 * (q >> 1) + 4 * (q & 1) + (e & 3) + 8 * (e >> 2);
}

// Byte offsets inside the LDS tiles (XOR swizzles keep the 16-byte lane
// accesses of both the staging writes and the MFMA operand reads spread over
// all banks).
__device__ __forceinline__ int k_off(int key, int chunk) {
  return key * kKRowBytes + ((chunk ^ (key & 7)) << 4);
}
__device__ __forceinline__ int vt_off(int q, int col) {
  return q * (kLkv * 16) + (((col & ~7) | ((col & 7) ^ ((col >> 3) & 7))) << 4);
}
__device__ __forceinline__ int p_off(int row, int q) {
  return row * 64 + ((q ^ ((row >> 1) & 3)) << 4);
}

template <bool FP8>
struct Stage;

template <>
struct Stage<false> {
  u32x4_t v[8];  // 8 keys x 8 latent columns
  u32x4_t r;     // one rope piece
};
template <>
struct Stage<true> {
  u32x2_t v[8];
  u32x2_t r;
};

// Element offsets (within the cache) of the rows of this thread's keys in a
// tile: 8 latent keys of chunk q and the rope key rk.  When page_size is a
// multiple of 32 the whole tile lies in one page and a single (uniform)
// block_table lookup serves it; otherwise every key looks up its own page,
// all lookups issued before any data load.
template <bool PAGED32>
__device__ __forceinline__ void tile_rows(const DecodeArgs& a, const int32_t* bt_row, int ts, int ke,
                                          int q, int rk, int64_t (&off)[9]) {
  const int ps = a.page_size;
  if constexpr (PAGED32) {
    const int page = ld_uniform(bt_row + (unsigned)ts / (unsigned)ps);
    const int64_t base = (int64_t)page * a.s_page + (int64_t)((unsigned)ts % (unsigned)ps) * a.s_tok;
#pragma unroll
    for (int e = 0; e < 8; ++e) off[e] = base + (int64_t)chunk_key(q, e) * a.s_tok;
    off[8] = base + (int64_t)rk * a.s_tok;
  } else {
    int pg[9];
    unsigned jj[9];
#pragma unroll
    for (int e = 0; e < 9; ++e) {
      const int j = ts + (e < 8 ? chunk_key(q, e) : rk);
      jj[e] = (unsigned)min(j, ke - 1);  // clamp: keys past ke are not loaded
      pg[e] = bt_row[jj[e] / (unsigned)ps];
    }
#pragma unroll
    for (int e = 0; e < 9; ++e) off[e] = (int64_t)pg[e] * a.s_page + (int64_t)(jj[e] % (unsigned)ps) * a.s_tok;
  }
}

// Issues the global loads of one tile: keys [ts, ts+32) of request b, clipped at ke.
template <bool FP8, bool PAGED32>
__device__ __forceinline__ void load_tile(const DecodeArgs& a, Stage<FP8>& st, int b, int ts, int ke,
                                          int tid) {
  const int32_t* bt_row = a.block_table + (int64_t)b * a.bt_s;
  const int q = tid >> 6, cg = tid & 63;
  const int rk = tid >> 3, rc = tid & 7;
  int64_t off[9];
  tile_rows<PAGED32>(a, bt_row, ts, ke, q, rk, off);
  if constexpr (!FP8) {
    const uint16_t* kvc = (const uint16_t*)a.kv_c + 8 * cg;
    const uint16_t* kpe = (const uint16_t*)a.k_pe + 8 * rc;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      st.v[e] = (ts + chunk_key(q, e) < ke) ? *(const u32x4_t*)(kvc + off[e]) : u32x4_t{0, 0, 0, 0};
    st.r = (ts + rk < ke) ? *(const u32x4_t*)(kpe + off[8]) : u32x4_t{0, 0, 0, 0};
  } else {
    const uint8_t* kvc = (const uint8_t*)a.kv_c + 8 * cg;
    const uint8_t* kpe = (const uint8_t*)a.k_pe + 8 * rc;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      st.v[e] = (ts + chunk_key(q, e) < ke) ? *(const u32x2_t*)(kvc + off[e]) : u32x2_t{0, 0};
    st.r = (ts + rk < ke) ? *(const u32x2_t*)(kpe + off[8]) : u32x2_t{0, 0};
  }
}

__device__ __forceinline__ u32x4_t widen8(u32x2_t w) {
  const u32x2_t lo = fp8x4_to_bf16x4(w[0]);
  const u32x2_t hi = fp8x4_to_bf16x4(w[1]);
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}

// Writes the staged tile into LDS: K rows (all 576 columns) and V^T.
template <bool FP8>
__device__ __forceinline__ void store_tile(char* smem, int stage, const Stage<FP8>& st, int tid) {
  char* kt = smem + kKOff + stage * kKStageBytes;
  char* vt = smem + kVtOff + stage * kVtStageBytes;
  const int q = tid >> 6, cg = tid & 63;
  u32x4_t r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (FP8) r[e] = widen8(st.v[e]); else r[e] = st.v[e];
    *(u32x4_t*)(kt + k_off(chunk_key(q, e), cg)) = r[e];
  }
  {
    const int rk = tid >> 3, rc = tid & 7;
    u32x4_t rr;
    if constexpr (FP8) rr = widen8(st.r); else rr = st.r;
    *(u32x4_t*)(kt + k_off(rk, 64 + rc)) = rr;
  }
  // 8x8 transpose: out[c] holds column 8*cg+c of the 8 keys of chunk q.
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    u32x4_t o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t x = r[2 * k][c >> 1], y = r[2 * k + 1][c >> 1];
      o[k] = (c & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
    }
    *(u32x4_t*)(vt + vt_off(q, 8 * cg + c)) = o;
  }
}

}  // namespace

template <bool FP8, bool PAGED32, int NRB>
__global__ __launch_bounds__(256, 1) void mla_decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l32 = l & 31, hh = l >> 5;

  // Workgroups are dealt round-robin to the 8 XCDs; keep the head groups of
  // one part on one XCD so that they share its L2 for the part's keys.
  const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const int hg = slot % a.head_groups;
  const int part = xcd + 8 * (slot / a.head_groups);
  if (part >= a.num_parts) return;

  const int R = a.Sq * a.N;
  const int row0 = hg * kGroupRows;
  const int RG = min(kGroupRows, R - row0);  // rows of this group; NRB = ceil(RG / 32) or more

  const int s_beg = ld_uniform(a.part_begin + part), s_end = ld_uniform(a.part_begin + part + 1);
  const int32_t* segs = a.segs;  // [num_segs][4]: req, kv_start, kv_end, partial

  Stage<FP8> st;
  int stage = 0;
  bool have = false;  // st holds the next tile to store

  float* ell_l = (float*)(smem + kEllOff);
  int* flag_l = (int*)(smem + kFlagOff);

  const int qrow_loc = 32 * w + l32;  // this lane's query row in QK^T (waves w < NRB)
  const bool qk_wave = w < NRB;

  for (int si = s_beg; si < s_end; ++si) {
    const int b = ld_uniform(segs + 4 * si), ks = ld_uniform(segs + 4 * si + 1);
    const int ke = ld_uniform(segs + 4 * si + 2), pidx = ld_uniform(segs + 4 * si + 3);
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
        lim = min(ke, L - (a.Sq - 1) + t);
      } else {
#pragma unroll
        for (int k = 0; k < 36; ++k) qr[k] = u32x4_t{0, 0, 0, 0};
      }
    }

    float m_ref = -INFINITY;  // reference max of this row (log2 units)
    float m_seen = -INFINITY; // largest logit seen so far
    float l_run = 0.f;
    f32x16_t O[4][NRB];
    for (;;) {  // one pass over the segment; repeated only after a restart request
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NRB; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) O[i][j][v] = 0.f;
      l_run = 0.f;
      bool restart = false;

      for (int ts = ks; ts < ke; ts += kTile) {
        if (!have) load_tile<FP8, PAGED32>(a, st, b, ts, ke, tid);
        store_tile<FP8>(smem, stage, st, tid);
        // Prefetch the next tile: later in this segment or the first tile of the
        // next segment that has keys.
        have = false;
        if (ts + kTile < ke) {
          load_tile<FP8, PAGED32>(a, st, b, ts + kTile, ke, tid);
          have = true;
        } else {
          for (int sn = si + 1; sn < s_end; ++sn) {
            const int nb = ld_uniform(segs + 4 * sn), nks = ld_uniform(segs + 4 * sn + 1);
            const int nke = ld_uniform(segs + 4 * sn + 2);
            if (nke > nks) {
              load_tile<FP8, PAGED32>(a, st, nb, nks, nke, tid);
              have = true;
              break;
            }
          }
        }
        __syncthreads();

        if (qk_wave) {
          const char* kt = smem + kKOff + stage * kKStageBytes;
          f32x16_t sacc;
#pragma unroll
          for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
          for (int k = 0; k < 36; ++k) {
            const u32x4_t kf = *(const u32x4_t*)(kt + k_off(l32, 2 * k + hh));
            sacc = mfma32(kf, qr[k], sacc);
          }
          float mx = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = ts + 8 * (v >> 2) + 4 * hh + (v & 3);
            sacc[v] = (j < lim) ? sacc[v] * a.qk_scale_log2 : -INFINITY;
            mx = fmaxf(mx, sacc[v]);
          }
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          m_seen = fmaxf(m_seen, mx);
          if (m_ref == -INFINITY) m_ref = mx;  // first visible keys: O and l are still 0
          const bool over = mx > m_ref + kMaxOvershoot;
          const bool dead = (m_ref == -INFINITY);
          float psum = 0.f;
          uint32_t pk[8];
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            const float p0 = dead ? 0.f : fast_exp2(sacc[v] - m_ref);
            const float p1 = dead ? 0.f : fast_exp2(sacc[v + 1] - m_ref);
            psum += p0 + p1;
            pk[v >> 1] = pack_bf16x2(p0, p1);
          }
          psum += __shfl_xor(psum, 32);
          l_run += psum;
          // keys 8s'..8s'+7 of this lane's accumulator form P chunk q = 2s' + hh
          *(u32x4_t*)(smem + kPOff + p_off(qrow_loc, hh)) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
          *(u32x4_t*)(smem + kPOff + p_off(qrow_loc, 2 + hh)) = u32x4_t{pk[4], pk[5], pk[6], pk[7]};
          const bool any = __any(over);
          if (l == 0) flag_l[w] = any ? 1 : 0;
        }
        __syncthreads();

#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) restart |= (flag_l[rb] != 0);
        if (restart) break;  // uniform over the workgroup

        // O^T[cols of wave w][rows] += V^T . P^T
        {
          const char* vt = smem + kVtOff + stage * kVtStageBytes;
          u32x4_t pf[NRB][2];
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int s = 0; s < 2; ++s)
              pf[rb][s] = *(const u32x4_t*)(smem + kPOff + p_off(32 * rb + l32, 2 * s + hh));
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const int col = 128 * w + 32 * cb + l32;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const u32x4_t vf = *(const u32x4_t*)(vt + vt_off(2 * s + hh, col));
#pragma unroll
              for (int rb = 0; rb < NRB; ++rb) O[cb][rb] = mfma32(vf, pf[rb][s], O[cb][rb]);
            }
          }
        }
        stage ^= 1;
      }
      if (!restart) break;
      // Raise every row's reference to the largest logit seen and start over.
      m_ref = m_seen;
      stage ^= 1;
      have = false;
      __syncthreads();  // nobody still reads the flags or this stage
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
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int rl = 32 * rb + l32;
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
            const int col = 128 * w + 32 * cb + 8 * g + 4 * hh;
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
            const int col = 128 * w + 32 * cb + 8 * g + 4 * hh;
            const f32x16_t& acc = O[cb][rb];
            *(f32x4_t*)(prow + col) =
                f32x4_t{acc[4 * g] * f, acc[4 * g + 1] * f, acc[4 * g + 2] * f, acc[4 * g + 3] * f};
          }
      }
    }
  }
}

template <bool FP8, bool PAGED32>
static hipError_t launch_nrb(const DecodeArgs& a, int nrb, dim3 grid, hipStream_t stream) {
  switch (nrb) {
    case 1: hipLaunchKernelGGL((mla_decode_kernel<FP8, PAGED32, 1>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((mla_decode_kernel<FP8, PAGED32, 2>), grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((mla_decode_kernel<FP8, PAGED32, 3>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((mla_decode_kernel<FP8, PAGED32, 4>), grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, bool fp8, hipStream_t stream) {
  // Every head group but the last has 128 rows; the last may be smaller, but a
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
