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
// Attention kernel.  One workgroup (4 waves) per (request, block of 128 queries, head);
// wave w owns queries 32w..32w+31, one per lane column.  Per tile of 32 keys:
//   S^T[key][query] = K[key][:] . Q[query][:]     (12 MFMAs 32x32x16, K from LDS)
//   online softmax per query (the 16 logits of a lane plus its partner lane l^32)
//   O^T[v][query]  += V^T[v][key] . P^T[key][query] (8 MFMAs, V^T from LDS)
// so every per-query quantity (maximum, row sum, rescale factor) is a per-lane scalar.
// K sits in LDS as [key][192] rows of 400 bytes and V transposed as [v][32 keys] rows of
// 72 bytes: both strides make the 16-lane (b128) and 32-lane (b64) reads of one MFMA
// operand hit distinct banks.  The next tile is loaded into registers while the current
// one is computed.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kPT = 32;          // keys per tile
constexpr int kKRow = 200;       // bf16 per K row in LDS (192 + 8 pad): 400 bytes
constexpr int kVRow = 36;        // bf16 per V^T row in LDS (32 keys + 4 pad): 72 bytes
constexpr int kPN = 128;         // P (k_nope / q_nope width)
constexpr int kPR = 64;          // R (rope width)
constexpr int kPV = 128;         // V (value width)

__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillAttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sk[kPT * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t sv[kPV * kVRow];
  const int b = blockIdx.z, h = blockIdx.y;
  const int qb = gridDim.x - 1 - blockIdx.x;  // longest (causal) blocks first
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

  // tile loads: K as 32 keys x 24 chunks of 16 B (3 per thread); V by threads 0..127 as
  // 4 keys x 8 values each (transposed on the way to LDS)
  u32x4_t rk[3], rv[4];
  auto load = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int u = tid + 256 * i, key = u / 24, c = u - 24 * key;
      const int j = kt * kPT + key;
      rk[i] = u32x4_t{0, 0, 0, 0};
      if (j < Sk) {
        const int64_t s = (int64_t)k0 + j;
        rk[i] = c < 16 ? *(const u32x4_t*)(a.k_nope + s * a.kn_s_tok + (int64_t)h * a.kn_s_head + 8 * c)
                       : *(const u32x4_t*)(a.k_pe + s * a.kp_s_tok + 8 * (c - 16));
      }
    }
    if (tid < 128) {
      const int kq = tid >> 4, vo = tid & 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kt * kPT + 4 * kq + r;
        rv[r] = u32x4_t{0, 0, 0, 0};
        if (j < Sk) rv[r] = *(const u32x4_t*)(a.v + ((int64_t)k0 + j) * a.v_s_tok + (int64_t)h * a.v_s_head + 8 * vo);
      }
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int u = tid + 256 * i, key = u / 24, c = u - 24 * key;
      *(u32x4_t*)(sk + key * kKRow + 8 * c) = rk[i];
    }
    if (tid < 128) {
      const int kq = tid >> 4, vo = tid & 15;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int sh = 16 * (c & 1);
        const uint32_t e0 = (rv[0][c >> 1] >> sh) & 0xFFFFu, e1 = (rv[1][c >> 1] >> sh) & 0xFFFFu;
        const uint32_t e2 = (rv[2][c >> 1] >> sh) & 0xFFFFu, e3 = (rv[3][c >> 1] >> sh) & 0xFFFFu;
        *(u32x2_t*)(sv + (8 * vo + c) * kVRow + 4 * kq) = u32x2_t{e0 | (e1 << 16), e2 | (e3 << 16)};
      }
    }
  };

  f32x16_t o[4];
#pragma unroll
  for (int vb = 0; vb < 4; ++vb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[vb][e] = 0.f;
  float m = -INFINITY, lsum = 0.f;  // log2-domain running maximum; this half's row sum

  if (ntiles > 0) load(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();  // the previous tile's reads are done
    store();
    __syncthreads();
    if (kt + 1 < ntiles) load(kt + 1);  // in flight during this tile's math

    f32x16_t s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      const u32x4_t kf = *(const u32x4_t*)(sk + l32 * kKRow + 16 * ks + 8 * hh);
      s = mfma32(kf, qf[ks], s);
    }
    // lane holds keys 8 gq + 4 hh + e of the tile (index 4 gq + e) for query qi
    float x[16];
    float mx = -INFINITY;
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const int j = kt * kPT + 8 * (idx >> 2) + 4 * hh + (idx & 3);
      x[idx] = (j <= qlim && j < Sk) ? s[idx] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[idx]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);  // 0 while m is -inf
    float ps = 0.f;
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      x[idx] = exp2f(x[idx] - m_use);
      ps += x[idx];
    }
    lsum = lsum * alpha + ps;
    m = m_new;
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[vb][e] *= alpha;
    // P^T operand of k-step ss: k-slot 8 hh + c <-> key 16 ss + 4 hh + c (c < 4) and
    // 16 ss + 8 + 4 hh + (c - 4) (c >= 4): accumulator indices 8 ss .. 8 ss + 7
    u32x4_t pb[2];
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
      pb[ss] = u32x4_t{pack_bf16x2(x[8 * ss], x[8 * ss + 1]), pack_bf16x2(x[8 * ss + 2], x[8 * ss + 3]),
                       pack_bf16x2(x[8 * ss + 4], x[8 * ss + 5]), pack_bf16x2(x[8 * ss + 6], x[8 * ss + 7])};
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const uint16_t* vr = sv + (32 * vb + l32) * kVRow + 16 * ss + 4 * hh;
        const u32x2_t lo = *(const u32x2_t*)vr, hi = *(const u32x2_t*)(vr + 8);
        o[vb] = mfma32(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pb[ss], o[vb]);
      }
  }

  // epilogue: o = O / l (bf16), lse = ln sum exp (scale included); no key -> 0, -inf
  const float lrow = lsum + __shfl_xor(lsum, 32);
  if (!qvalid) return;
  const int64_t t = (int64_t)q0 + qi;
  const float f = lrow > 0.f ? 1.f / lrow : 0.f;
  if (a.lse && hh == 0) a.lse[t * a.N + h] = lrow > 0.f ? (m + log2f(lrow)) * kLn2 : -INFINITY;
  uint16_t* orow = a.o + t * a.o_s_tok + (int64_t)h * a.o_s_head;
#pragma unroll
  for (int vb = 0; vb < 4; ++vb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int v = 32 * vb + 8 * gq + 4 * hh;
      *(u32x2_t*)(orow + v) = u32x2_t{pack_bf16x2(o[vb][4 * gq] * f, o[vb][4 * gq + 1] * f),
                                      pack_bf16x2(o[vb][4 * gq + 2] * f, o[vb][4 * gq + 3] * f)};
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
  const dim3 grid((max_q + 127) / 128, a.N, B);
  hipLaunchKernelGGL(prefill_attn_kernel, grid, dim3(256), 0, stream, a);
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
