// Kernel argument blocks and launchers (host <-> device interface inside the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace mla {

struct DecodeArgs {
  const uint16_t* q_nope;  // [T, N, 512] bf16
  int64_t q_nope_s_tok, q_nope_s_head;
  const uint16_t* q_pe;    // [T, N, 64] bf16
  int64_t q_pe_s_tok, q_pe_s_head;
  const void* kv_c;        // cache base for columns 0..511 (bf16 or e4m3fn)
  const void* k_pe;        // cache base for columns 512..575
  int64_t s_page, s_tok;   // cache strides in elements
  const int32_t* block_table;
  int64_t bt_s;
  const int32_t* seq_lens;
  const int32_t* part_begin;  // [num_parts + 1]
  const int32_t* segs;        // [num_segs][4]: req, kv_start, kv_end, partial
  uint16_t* o;                // [T, N, 512] bf16
  int64_t o_s_tok, o_s_head;
  float* lse;                 // [T, N] or null
  void* ws_o;                 // [partials, Sq*N rounded up to 32, 512] fp16, scaled (blocked)
  float* ws_lse;              // [partials, Sq*N]
  float* ws_l;                // [partials, Sq*N]: row sums / kv_scale, times the block's scale
  const uint8_t* q8;          // fp8 queries [T, N, 576] e4m3fn (null: bf16 q_nope / q_pe)
  int64_t q8_s_tok, q8_s_head;  // bytes
  float qk_scale_log2;        // scale * kv_scale (* q_scale for fp8 queries) * log2(e)
  float out_scale;            // kv_scale
  int32_t Sq, N, page_size, num_parts, head_groups;
};

struct MergeArgs {
  const int32_t* reduce;  // [n_reduce][3]: req, first partial, count
  int32_t n_reduce;
  const void* ws_o;
  const float* ws_lse;
  const float* ws_l;
  uint16_t* o;
  int64_t o_s_tok, o_s_head;
  float* lse;
  int32_t Sq, N;
};

struct QuantArgs {
  const uint16_t* ql;   // [T, N, 512] bf16
  int64_t ql_s_tok, ql_s_head;
  const uint16_t* qpe;  // [T, N, 64] bf16
  int64_t qpe_s_tok, qpe_s_head;
  uint8_t* q8;          // [T, N, 576] e4m3fn
  int64_t q8_s_tok, q8_s_head;
  float inv_scale;      // 1 / q_scale, rounded once to fp32
  int32_t T, N;
};

struct CacheWriteArgs {
  const uint16_t* kv_c;  // [T, 512] bf16
  int64_t kv_c_s_tok;
  const uint16_t* k_pe;  // [T, 64] bf16
  int64_t k_pe_s_tok;
  const int64_t* slot_mapping;  // [T]
  void* cache;                  // [num_pages, page_size, 576] bf16 or e4m3fn
  int64_t s_page, s_tok;        // elements
  float inv_scale;              // fp8: 1 / k_scale, rounded once to fp32
  int32_t T, page_size, num_pages;
};

hipError_t launch_decode(const DecodeArgs& a, bool fp8, bool qf8, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_concat_quant_q(const QuantArgs& a, hipStream_t stream);
hipError_t launch_split_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_merge_two(void* out, float* out_lse, const void* prefix_o, const float* prefix_lse,
                            const void* suffix_o, const float* suffix_lse, int64_t rows, int32_t D,
                            bool fp32, hipStream_t stream);
// C[h][m][n] = sum_k A[h][m][k] * B[h][n][k] in bf16 with fp32 accumulation.
// A: element (h,m,k) at h*a_sh + m*a_sm + k.  B: (h,n,k) at h*b_sh + n*b_sn + k*b_sk,
// with either b_sk == 1 (k-contiguous) or b_sn == 1 (n-contiguous).
// C: (h,m,n) at h*c_sh + m*c_sm + n.
struct GemmArgs {
  const uint16_t* A;
  int64_t a_sh, a_sm;
  const uint16_t* B;
  int64_t b_sh, b_sn, b_sk;
  uint16_t* C;
  int64_t c_sh, c_sm;
  int32_t H, M, Nn, K;
};
hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream);
// kv_b_proj: C0[s][n] = sum_k A[s][k] B0[k][n] (n < N0) and C1 likewise with B1 (n < N1),
// bf16 with fp32 accumulation; A row stride a_s, B and C rows contiguous (stride N0 / N1).
// K must be a multiple of 32 and N0, N1 multiples of 8 (>= 8); tile counts set by the launcher.
struct KvbArgs {
  const uint16_t* A;
  int64_t a_s;
  const uint16_t* B0;
  const uint16_t* B1;
  uint16_t* C0;
  uint16_t* C1;
  int32_t N0, N1, M, K;
  int32_t mt, nt0, nt, per_xcd;
};
hipError_t launch_kvb_gemm(KvbArgs g, hipStream_t stream);
hipError_t launch_gather_rows(const int32_t* block_table, int64_t bt_s, const int32_t* seq_lens,
                              const int64_t* offsets, int32_t B, int32_t page_size, int64_t* rows,
                              hipStream_t stream);

// Prefill attention (compute-friendly MLA): per head, q = [q_nope | q_pe] (P+R = 192),
// k = [k_nope | k_pe] with k_pe shared by all heads, v (V = 128).  Request b owns queries
// cu_q[b]..cu_q[b+1]-1 and keys cu_k[b]..cu_k[b+1]-1; causal: query i of the request
// sees keys j <= i + Sk - Sq.  Strides in elements; lse [T, N] (t*N + h) or null.
struct PrefillAttnArgs {
  const uint16_t* q_nope;
  int64_t qn_s_tok, qn_s_head;
  const uint16_t* q_pe;
  int64_t qp_s_tok, qp_s_head;
  const uint16_t* k_nope;
  int64_t kn_s_tok, kn_s_head;
  const uint16_t* k_pe;
  int64_t kp_s_tok;
  const uint16_t* v;
  int64_t v_s_tok, v_s_head;
  const int32_t* cu_q;
  const int32_t* cu_k;
  uint16_t* o;
  int64_t o_s_tok, o_s_head;
  float* lse;
  // optional running state (same layouts as o / lse, may alias them): the output becomes
  // the LSE merge of that state with this launch's attention
  const uint16_t* prev_o;
  const float* prev_lse;
  float scale_log2;  // scale * log2(e)
  int32_t N, causal;
  int32_t q_blocks, items, per_xcd;  // set by the launcher
};
// Context gather of one chunk: output row r (request b: cu[b] <= r < cu[b+1]) is
// context position starts[b] + r - cu[b], as bf16 [kv_c 512] and [k_pe 64] rows.
struct GatherArgs {
  const void* kv_c;  // cache base, columns 0..511 (bf16 or e4m3fn)
  const void* k_pe;  // cache base, columns 512..575
  int64_t s_page, s_tok;  // elements
  const int32_t* block_table;
  int64_t bt_s;
  const int32_t* starts;  // [B]
  const int32_t* cu;      // [B + 1]
  uint16_t* out_kv_c;
  int64_t okv_s;
  uint16_t* out_k_pe;
  int64_t ope_s;
  float kv_scale;
  int64_t total;
  int32_t B, page_size;
};
hipError_t launch_prefill_attn(const PrefillAttnArgs& a, int32_t B, int32_t max_q, hipStream_t stream);
hipError_t launch_gather_ctx(const GatherArgs& a, bool fp8, hipStream_t stream);

// fp8 batched GEMM: C[h][m][n] = w_scale * sum_g d[h][m][g] sum_{k in g} A8[h][m][k] W8[h][n][k],
// A bf16 (h,m,k) at h*a_sh + m*a_sm + k, quantised per (m, group of 128 k) in the kernel;
// B e4m3fn (h,n,k) at h*b_sh + n*b_sn + k (bytes); C bf16 (h,m,n) at h*c_sh + m*c_sm + n.
struct Bmm8Args {
  const uint16_t* A;
  int64_t a_sh, a_sm;
  const uint8_t* B;
  int64_t b_sh, b_sn;
  uint16_t* C;
  int64_t c_sh, c_sm;
  const float* w_scale;  // device, one value
  int32_t H, M, Nn, K;
};
hipError_t launch_bmm8(const Bmm8Args& g, hipStream_t stream);
hipError_t launch_quant_weight(const uint16_t* W, int32_t Lkv, int32_t N, int32_t X, int32_t which,
                               uint8_t* out, float* w_scale, hipStream_t stream);

}  // namespace mla
