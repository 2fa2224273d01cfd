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
// Attention kernel.  One workgroup (4 waves, two workgroups per CU) per (request, head,
// block of 128 queries), dealt to the XCDs so that the query blocks of one head share an
// L2; wave w owns queries 32w..32w+31, one per lane column.  Per tile of 32 keys:
//   S^T[key][query] = K[key][:] . Q[query][:]     (12 MFMAs 32x32x16, K from LDS)
//   online softmax per query (the 16 logits of a lane plus its partner lane l^32)
//   O^T[v][query]  += V^T[v][key] . P^T[key][query] (8 MFMAs)
// so every per-query quantity (maximum, row sum, rescale factor) is a per-lane scalar.
// K sits in LDS as [key][192] rows of 400 bytes (the 16 lanes of a b128 read hit distinct
// banks) and V row-major as [key][128] rows of 272 bytes, read as V^T by transposing LDS
// reads (the 4 rows of one read land 64 bytes apart in the banks); the QK takes the K rows
// in a permuted key order so that P^T needs no shuffle.  The next tile is loaded into
// registers while the current one is computed.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kPT = 32;          // keys per tile
constexpr int kKRow = 200;       // bf16 per K row in LDS (192 + 8 pad): 400 bytes
constexpr int kVRow = 136;       // bf16 per V row in LDS (128 values + 8 pad): 272 bytes
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

__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillAttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sk[kPT * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t sv[kPT * kVRow];
  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin by launch index, so
  // launch index L takes work item (L % 8) * per + L / 8.  Each XCD then runs a contiguous
  // range of (request, head, query block) items: the query blocks of one head share that
  // XCD's L2 for their K and V tiles instead of each XCD streaming every head.
  const int L = blockIdx.x;
  const int item = (L & 7) * a.per_xcd + (L >> 3);
  if (item >= a.items) return;  // (whole workgroup; the launch is padded to 8 * per_xcd)
  const int nqb = a.q_blocks;
  const int qb = nqb - 1 - item % nqb;  // longest (causal) blocks first
  const int h = (item / nqb) % a.N, b = item / nqb / a.N;
  const int q0 = a.cu_q[b], Sq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], Sk = a.cu_k[b + 1] - k0;
  if (128 * qb >= Sq) return;  // (whole workgroup)
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l32 = l & 31, hh = l >> 5;
  const int qi = 128 * qb + 32 * w + l32;  // this lane's query within the request
  const bool qvalid = qi < Sq;
  // keys the workgroup needs: causal query i sees keys j <= i + Sk - Sq
  const int qlast = min(Sq, 128 * qb + 128) - 1;
  const int nkeys = a.causal ? max(0, min(Sk, qlast + Sk - Sq + 1)) : Sk;
  const int ntiles = (nkeys + kPT - 1) / kPT;
  const int qlim = a.causal ? qi + Sk - Sq : Sk - 1;  // last key this lane's query sees
  // tiles below this key count need no mask for any query of the workgroup
  const int unmasked = a.causal ? max(0, min(Sk, 128 * qb + Sk - Sq + 1)) : Sk;

  // queries: k-step ks covers dims 16 ks + 8 hh .. +7 (q_nope for ks < 8, q_pe after)
  u32x4_t qf[12];
  {
    const int64_t t = (int64_t)q0 + (qvalid ? qi : 0);
    const uint16_t* qn = a.q_nope + t * a.qn_s_tok + (int64_t)h * a.qn_s_head + 8 * hh;
    const uint16_t* qp = a.q_pe + t * a.qp_s_tok + (int64_t)h * a.qp_s_head + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      qf[ks] = u32x4_t{0, 0, 0, 0};
      if (qvalid) qf[ks] = ks < 8 ? *(const u32x4_t*)(qn + 16 * ks) : *(const u32x4_t*)(qp + 16 * (ks - 8));
    }
  }

  // Tile loads.  K: thread t covers key t / 8 of the tile, chunks 3 (t % 8) .. +2 of its
  // 24 (16 of k_nope, 8 of k_pe).  V: threads 0..127 cover 4 keys x 8 values each, which
  // are transposed on the way to LDS.  Row pointers advance by one tile per load.
  const int kkey = tid >> 3, kc0 = 3 * (tid & 7);
  const int vkey = tid >> 4, vc = tid & 15;  // V: keys vkey and vkey + 16, chunk vc of 16
  // Workgroup-uniform tile bases (advanced by one tile per load) and fixed 32-bit lane
  // offsets, so that the loads take the scalar-base form and need no 64-bit lane math.
  const uint16_t* kn_base = a.k_nope + (int64_t)k0 * a.kn_s_tok + (int64_t)h * a.kn_s_head;
  const uint16_t* kp_base = a.k_pe + (int64_t)k0 * a.kp_s_tok;
  const uint16_t* v_base = a.v + (int64_t)k0 * a.v_s_tok + (int64_t)h * a.v_s_head;
  // byte offsets (a zero-extended 32-bit lane offset on a uniform base is the scalar-base form)
  const uint32_t kn_off = (uint32_t)(2 * kkey * a.kn_s_tok), kp_off = (uint32_t)(2 * kkey * a.kp_s_tok);
  const uint32_t v_off0 = (uint32_t)(2 * (vkey * a.v_s_tok + 8 * vc)), v_off1 = v_off0 + (uint32_t)(32 * a.v_s_tok);
  const int64_t step_n = (int64_t)kPT * a.kn_s_tok, step_p = (int64_t)kPT * a.kp_s_tok;
  const int64_t step_v = (int64_t)kPT * a.v_s_tok;
  u32x4_t rk[3], rv[2];
  auto load = [&](int kt) __attribute__((always_inline)) {
    const bool full = kt * kPT + kPT <= Sk;  // (uniform) every key of the tile exists
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int c = kc0 + i;
      rk[i] = u32x4_t{0, 0, 0, 0};
      if (full || kt * kPT + kkey < Sk)
        rk[i] = c < 16 ? *(const u32x4_t*)((const char*)kn_base + (kn_off + 16u * c))
                       : *(const u32x4_t*)((const char*)kp_base + (kp_off + 16u * (c - 16)));
    }
    if (full || kt * kPT + vkey < Sk) rv[0] = *(const u32x4_t*)((const char*)v_base + v_off0);
    else rv[0] = u32x4_t{0, 0, 0, 0};
    if (full || kt * kPT + vkey + 16 < Sk) rv[1] = *(const u32x4_t*)((const char*)v_base + v_off1);
    else rv[1] = u32x4_t{0, 0, 0, 0};
    kn_base += step_n;
    kp_base += step_p;
    v_base += step_v;
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 3; ++i) *(u32x4_t*)(sk + kkey * kKRow + 8 * (kc0 + i)) = rk[i];
#pragma unroll
    for (int r = 0; r < 2; ++r) *(u32x4_t*)(sv + (vkey + 16 * r) * kVRow + 8 * vc) = rv[r];
  };

  f32x16_t o[4];
#pragma unroll
  for (int vb = 0; vb < 4; ++vb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[vb][e] = 0.f;
  // Softmax state in log2 units: p = 2^(c s - m) against a reference maximum m that only
  // moves when a logit exceeds it by more than kRescaleAt (p then stays below 2^8), so O
  // is rescaled rarely; lsum is this half's row sum.
  float m = -INFINITY, lsum = 0.f;
  const float cs = a.scale_log2;
  const int krow = pi_key(l32);  // K row this lane feeds to the QK MFMA
  // transposing-read address of this lane (elements): row hh + 4((l % 16) / 4), columns
  // 16 ((l / 16) % 2) + 4 (l % 4) of a 32-value block; k-step ss adds 16 rows, the second
  // read of a k-step 2 rows, value block vb 32 columns
  const int vtr = (hh + 4 * ((l & 15) >> 2)) * kVRow + 16 * ((l >> 4) & 1) + 4 * (l & 3);

  auto tile = [&](int kt) __attribute__((always_inline)) {
    // all K fragments of the tile are read before the MFMA chain starts, so that no MFMA
    // waits for an LDS round trip
    u32x4_t kf[12];
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) kf[ks] = *(const u32x4_t*)(sk + krow * kKRow + 16 * ks + 8 * hh);
    f32x16_t s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) s = mfma32(kf[ks], qf[ks], s);
    u32x4_t vf[8];  // V^T fragments (value block i / 2, k-step i % 2), read while the softmax runs
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t* p0 = sv + vtr + 16 * (i & 1) * kVRow + 32 * (i >> 1);
      vf[i] = read_vt(p0, p0 + 2 * kVRow);
    }
    // lane holds S^T rows 8 gq + 4 hh + e (index 4 gq + e), tile keys pi of those, for query qi
    if (kt * kPT + kPT > unmasked) {  // (uniform) a tile on the diagonal or past Sk
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const int j = kt * kPT + pi_key(8 * (idx >> 2) + 4 * hh + (idx & 3));
        if (j > qlim || j >= Sk) s[idx] = -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int idx = 1; idx < 16; ++idx) mx = fmaxf(mx, s[idx]);
    mx = half_max(mx) * cs;  // scale > 0: the maximum of the scaled logits
    if (__any(mx > m + kRescaleAt)) {
      const float m_new = mx > m + kRescaleAt ? mx : m;
      const float alpha = m_new == m ? 1.f : fast_exp2(m - m_new);  // 0 while m is -inf
      lsum *= alpha;
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[vb][e] *= alpha;
      m = m_new;
    }
    const float m_use = m == -INFINITY ? 0.f : m;  // a row with no key yet: every p is 0
    float x[16];
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      x[idx] = fast_exp2(fmaf(s[idx], cs, -m_use));  // v_exp_f32: results below 2^-126 flush to 0
      lsum += x[idx];
    }
    // P^T operand of k-step ss: accumulator indices 8 ss .. 8 ss + 7, which hold keys
    // 16 ss + hh + 4e and 16 ss + 2 + hh + 4e, the keys of the two transposing reads
    u32x4_t pb[2];
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
      pb[ss] = u32x4_t{pack_bf16x2(x[8 * ss], x[8 * ss + 1]), pack_bf16x2(x[8 * ss + 2], x[8 * ss + 3]),
                       pack_bf16x2(x[8 * ss + 4], x[8 * ss + 5]), pack_bf16x2(x[8 * ss + 6], x[8 * ss + 7])};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i >> 1] = mfma32(vf[i], pb[i & 1], o[i >> 1]);
  };

  // the next tile is in registers while this one is stored and computed
  if (ntiles > 0) load(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();  // the previous tile's reads are done
    store();
    __syncthreads();
    if (kt + 1 < ntiles) load(kt + 1);
    tile(kt);
  }

  // epilogue: o = O / l (bf16), lse = ln sum exp (scale included); no key -> 0, -inf.
  // With a running state (prev_o, prev_lse) the output is its LSE merge with this result:
  // m = max(lse_p, lse), o = (e^(lse_p - m) o_p + e^(lse - m) o) / z, lse = m + ln z.
  const float lrow = half_sum(lsum);
  if (!qvalid) return;
  const int64_t t = (int64_t)q0 + qi;
  const float lse_new = lrow > 0.f ? (m + fast_log2(lrow)) * kLn2 : -INFINITY;
  float f_new = lrow > 0.f ? 1.f / lrow : 0.f, f_prev = 0.f, lse_out = lse_new;
  uint16_t* orow = a.o + t * a.o_s_tok + (int64_t)h * a.o_s_head;
  const uint16_t* prow = a.prev_o ? a.prev_o + t * a.o_s_tok + (int64_t)h * a.o_s_head : nullptr;
  if (prow) {
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
  if (a.lse && hh == 0) a.lse[t * a.N + h] = lse_out;
#pragma unroll
  for (int vb = 0; vb < 4; ++vb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int v = 32 * vb + 8 * gq + 4 * hh;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = o[vb][4 * gq + e] * f_new;
      if (prow) {  // read before this lane's own write of the same 8 bytes (o may alias prev_o)
        const u32x2_t pv2 = *(const u32x2_t*)(prow + v);
        y[0] += f_prev * bf16_to_f32((uint16_t)(pv2[0] & 0xFFFF));
        y[1] += f_prev * bf16_to_f32((uint16_t)(pv2[0] >> 16));
        y[2] += f_prev * bf16_to_f32((uint16_t)(pv2[1] & 0xFFFF));
        y[3] += f_prev * bf16_to_f32((uint16_t)(pv2[1] >> 16));
      }
      *(u32x2_t*)(orow + v) = u32x2_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    }
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
  g.q_blocks = (max_q + 127) / 128;
  g.items = g.q_blocks * a.N * B;
  g.per_xcd = (g.items + 7) / 8;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(8 * g.per_xcd), dim3(256), 0, stream, g);
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
