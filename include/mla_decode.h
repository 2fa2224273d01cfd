/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) MLA paged-decode library.
 *
 * The operation is DeepSeek-style Multi-Head Latent Attention decode in its
 * absorbed ("data-movement friendly") form, as defined in the module
 * docstring of vLLM's v1/attention/backends/mla/common.py, section
 * "Data-Movement Friendly Approach": the query is absorbed through W_UK
 * (ql_nope = q_nope . W_UK), every head attends over the same latent cache
 * rows [kv_c | k_pe] (an MQA with QK head dim Lkv+R = 576 and V head dim
 * Lkv = 512), and the latent output is up-projected through W_UV.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers unless the name ends in _host.
 *    Tensors are caller-owned; run/absorb/up/merge allocate nothing.
 *  - bf16 tensors are passed as raw 16-bit storage (void*), fp8 as bytes.
 *  - Strides are in ELEMENTS of the tensor's own type.
 *  - Every call is enqueued on the caller's HIP stream and returns without a
 *    host synchronisation.  Device data (block_table entries, seq_lens) is a
 *    precondition and is not read back: block_table[b][j] must be a valid page
 *    in [0, num_pages) for every j < ceil(seq_lens[b] / page_size); entries
 *    past that are never read (they may hold -1).
 *  - Return value: MLA_OK or a negative mla_status.  Nothing throws or aborts
 *    across the ABI.  mla_last_error() gives text for the calling thread's
 *    last non-OK status.
 *  - Dimensions supported: Lkv = 512 and R = 64 only (head size 576, the only
 *    MLA head size the vLLM backends accept); 1 <= N <= 128 query heads;
 *    1 <= Sq <= 8 query tokens per request, uniform over the batch (the ROCm
 *    backend builds qo_indptr with a uniform query length); any page_size >= 1.
 *    KV cache bf16 or OCP float8 e4m3fn; queries and latent output bf16;
 *    LSE fp32, natural log, including the softmax scale.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* null pointer, bad size or stride, inconsistent arguments */
  MLA_ERR_UNSUPPORTED = -2, /* valid request outside what the library implements     */
  MLA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the plan requires      */
  MLA_ERR_HIP = -4,         /* a HIP runtime call failed; text from hipGetErrorString   */
  MLA_ERR_INTERNAL = -5
} mla_status;

typedef enum { MLA_DT_BF16 = 0, MLA_DT_FP8_E4M3FN = 1, MLA_DT_FP32 = 2 } mla_dtype;

/* Opaque, library-owned plan.  hipStream_t is passed as void* so that this
 * header does not depend on the HIP headers. */
typedef struct mla_plan_s* mla_plan;

/*
 * mla_decode_plan -- split-KV work plan for one batch (host work, once per
 * batch, reused by every layer that decodes the same batch).
 *
 * The pages compute this schedule ahead of the forward pass and keep it off
 * the per-layer path (rocm_aiter_mla, AiterMLAMetadataBuilder: persistent
 * work / reduce maps filled per batch; mla/common.py metadata builder: avoid
 * GPU-to-CPU syncs).  The rule is this library's own: the keys of all
 * requests, in granules of 64, are dealt to at most num_cus / head_groups
 * parts of near-equal cost; a request cut between parts is computed as
 * partial states merged by LSE (the combiner of the mla/common.py docstring,
 * "Chunked Prefill").  Rows of a request are Sq*N (row r = t*N + h); they are
 * processed in head groups of up to 128 consecutive rows.
 *
 *  seq_lens_host      [B] host int32, keys per request (>= 0), including the
 *                     Sq new tokens; query row t of a request sees keys
 *                     j < seq_len - (Sq-1) + t (rocm_aiter_mla,
 *                     AiterMLAImpl.forward_mqa, multi-token verify).
 *  B, Sq, N, Lkv, R   batch, query tokens per request, heads, latent and rope width.
 *  page_size          tokens per cache page (>= 1).
 *  max_pages_per_req  columns of block_table; seq_len <= max_pages_per_req*page_size.
 *  kv_dtype           MLA_DT_BF16 or MLA_DT_FP8_E4M3FN.
 *  num_cus            compute units to plan for; <= 0 queries the current device.
 *  stream             hipStream_t on which the plan's device upload is enqueued.
 *  plan_out           receives the plan (owned by the library until mla_plan_destroy).
 *  workspace_bytes_out  receives the workspace size mla_decode_run needs (0 if no
 *                     request is split): the partial outputs of split requests (fp16,
 *                     scaled per 32-row block), their LSEs and row sums (fp32).
 * Errors: INVALID_ARG (null pointers, B < 1, negative seq_len, seq_len above 2^30
 * or beyond max_pages_per_req*page_size, page_size < 1), UNSUPPORTED (Lkv != 512,
 * R != 64, N outside [1,128], Sq outside [1,8], other kv_dtype), HIP.
 */
int mla_decode_plan(const int32_t* seq_lens_host, int32_t B, int32_t Sq, int32_t N, int32_t Lkv,
                    int32_t R, int32_t page_size, int32_t max_pages_per_req, int32_t kv_dtype,
                    int32_t num_cus, void* stream, mla_plan* plan_out,
                    size_t* workspace_bytes_out);

/* Waits for the plan's stream, then frees the plan.  NULL is accepted. */
int mla_plan_destroy(mla_plan plan);

/*
 * mla_decode_run -- latent attention of every query row over the paged cache.
 *
 * For request b, query row (t, h) and key j < n = max(0, L_b - (Sq-1) + t):
 *   row_j = block_table[b][j / page_size] * page_size + j % page_size
 *   s_j   = scale * kv_scale * (ql_nope[t,h] . kv_c[row_j] + q_pe[t,h] . k_pe[row_j])
 *   o_latent[t,h] = kv_scale * sum_j softmax(s)_j kv_c[row_j]
 *   lse[t,h]      = ln sum_j exp(s_j)
 * (mla/common.py docstring, "Data-Movement Friendly Approach": SDPA of
 * [ql_nope | q_pe] against [kv_c | k_pe] with value kv_c; the page expansion
 * of rocm_aiter_mla, AiterMLAMetadataBuilder._build_decode.)  kv_scale is the
 * per-tensor dequantisation scale of an fp8 cache (1 for bf16).  scale and
 * kv_scale must be finite and positive (MLA_ERR_INVALID_ARG otherwise).  A row
 * with n = 0 gets o_latent = 0 and lse = -inf.
 *
 *  q_nope    [B*Sq, N, 512] bf16, absorbed query ql_nope; token stride q_nope_s_tok, head stride q_nope_s_head.
 *  q_pe      [B*Sq, N, 64] bf16, strides q_pe_s_tok, q_pe_s_head.
 *  cache_kv_c / cache_k_pe  the latent cache [num_pages, page_size, 576] as two base
 *            pointers sharing strides (canonical: cache_k_pe = cache_kv_c + 512 elements);
 *            page stride cache_s_page, token stride cache_s_tok, dims contiguous.
 *  block_table [B, max_pages_per_req] int32, row stride block_table_s_req.
 *  seq_lens  [B] int32 device copy of the plan's seq_lens (must be equal).
 *  o_latent  [B*Sq, N, 512] bf16 output, strides o_s_tok, o_s_head.
 *  lse       [B*Sq, N] fp32 output (contiguous) or NULL.
 *  workspace device scratch of at least the plan's workspace_bytes (may be NULL if 0).
 * Errors: INVALID_ARG (nulls, bad strides, misaligned pointers: query and output
 * rows must be 16-byte aligned, cache rows 16-byte (bf16) or 8-byte (fp8)),
 * WORKSPACE, HIP.
 */
int mla_decode_run(mla_plan plan, const void* q_nope, int64_t q_nope_s_tok, int64_t q_nope_s_head,
                   const void* q_pe, int64_t q_pe_s_tok, int64_t q_pe_s_head,
                   const void* cache_kv_c, const void* cache_k_pe, int64_t cache_s_page,
                   int64_t cache_s_tok, int32_t num_pages, const int32_t* block_table,
                   int64_t block_table_s_req, const int32_t* seq_lens, float scale,
                   float kv_scale, void* o_latent, int64_t o_s_tok, int64_t o_s_head, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_attend / mla_decode_reduce -- the two phases of mla_decode_run,
 * for callers that schedule or time them separately (the persistent decode of
 * rocm_aiter_mla likewise runs attention over work items and then a reduce
 * over split requests).  attend takes exactly the arguments of mla_decode_run
 * and writes the final output of unsplit requests plus the partial states of
 * split ones into the workspace; reduce merges those partial states into
 * o_latent / lse.  reduce is a no-op when the plan splits nothing.  Running
 * attend then reduce on one stream is identical to mla_decode_run.
 */
int mla_decode_attend(mla_plan plan, const void* q_nope, int64_t q_nope_s_tok,
                      int64_t q_nope_s_head, const void* q_pe, int64_t q_pe_s_tok,
                      int64_t q_pe_s_head, const void* cache_kv_c, const void* cache_k_pe,
                      int64_t cache_s_page, int64_t cache_s_tok, int32_t num_pages,
                      const int32_t* block_table, int64_t block_table_s_req,
                      const int32_t* seq_lens, float scale, float kv_scale, void* o_latent,
                      int64_t o_s_tok, int64_t o_s_head, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);
int mla_decode_reduce(mla_plan plan, void* o_latent, int64_t o_s_tok, int64_t o_s_head, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_run_noalloc -- mla_decode_run for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and kernels, with the split partial states kept
 * in a static device array of the library instead of a caller's workspace.  It calls
 * no hipMalloc / hipFree and nothing that allocates.
 *
 * Arguments, ownership and errors are those of mla_decode_run without workspace /
 * workspace_bytes.  The static array holds 64 MiB (67108864 bytes) per device, for as
 * long as the process runs; a plan whose workspace_bytes exceeds it is rejected with
 * MLA_ERR_WORKSPACE before anything is enqueued.  Every call on a device shares that
 * device's array, and calls that overlap on one device (different streams, or host
 * threads) race on it; calls on one stream are ordered and safe.  Nothing in the array
 * needs clearing between calls: attend writes every partial state that reduce reads.
 */
int mla_decode_run_noalloc(mla_plan plan, const void* q_nope, int64_t q_nope_s_tok, int64_t q_nope_s_head,
                           const void* q_pe, int64_t q_pe_s_tok, int64_t q_pe_s_head, const void* cache_kv_c,
                           const void* cache_k_pe, int64_t cache_s_page, int64_t cache_s_tok, int32_t num_pages,
                           const int32_t* block_table, int64_t block_table_s_req, const int32_t* seq_lens,
                           float scale, float kv_scale, void* o_latent, int64_t o_s_tok, int64_t o_s_head,
                           float* lse, void* stream);

/*
 * mla_decode_run_q8 / mla_decode_attend_q8 -- mla_decode_run / mla_decode_attend for
 * an fp8 cache with an fp8 query: q8 = [ql_nope | q_pe] quantised with the static
 * per-tensor q_scale (mla_concat_quant_q; vLLM MLAAttention quantises the decode query
 * whenever the cache is fp8 and the backend takes a quantised query, and the ROCm
 * backend then runs with an fp8 query, rocm_aiter_mla page).  The logits are
 *   s_j = scale * q_scale * kv_scale * (q8[t,h] . cache[row_j])
 * in fp32 from exact fp8 products (the softmax scale takes q_scale together with the
 * cache scale, as the flashinfer page's bmm1_scale does); everything after the logits
 * is as in mla_decode_run (values widened to bf16, bf16 P.V, fp32 accumulation).
 *
 *  q8        [B*Sq, N, 576] float8 e4m3fn bytes; strides q8_s_tok, q8_s_head in bytes,
 *            multiples of 16, q8_s_head >= 576; 16-byte aligned.
 *  q_scale   finite and > 0.
 *  The plan must be for an fp8 cache (MLA_ERR_UNSUPPORTED otherwise).  All other
 *  arguments, ownership and errors as mla_decode_run; mla_decode_reduce completes
 *  attend_q8 as it completes attend.
 */
int mla_decode_run_q8(mla_plan plan, const void* q8, int64_t q8_s_tok, int64_t q8_s_head, float q_scale,
                      const void* cache_kv_c, const void* cache_k_pe, int64_t cache_s_page,
                      int64_t cache_s_tok, int32_t num_pages, const int32_t* block_table,
                      int64_t block_table_s_req, const int32_t* seq_lens, float scale, float kv_scale,
                      void* o_latent, int64_t o_s_tok, int64_t o_s_head, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);
int mla_decode_attend_q8(mla_plan plan, const void* q8, int64_t q8_s_tok, int64_t q8_s_head, float q_scale,
                         const void* cache_kv_c, const void* cache_k_pe, int64_t cache_s_page,
                         int64_t cache_s_tok, int32_t num_pages, const int32_t* block_table,
                         int64_t block_table_s_req, const int32_t* seq_lens, float scale, float kv_scale,
                         void* o_latent, int64_t o_s_tok, int64_t o_s_head, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * mla_absorb_q -- ql_nope[t,h,l] = sum_p q_nope[t,h,p] * W_UK[l,h,p].
 * mla/common.py docstring, "Data-Movement Friendly Approach" (einsum
 * "snh,lnh->snl"); the layer runs it as a per-head bmm (N,B,P)x(N,P,L)
 * (mla_attention, MLAAttention.forward_impl).  W_UK is the kv_b_proj slice
 * [Lkv, N, P] (mla_attention, process_weights_after_loading).
 *  q_nope [T, N, P] bf16 contiguous; W_UK [Lkv, N, P] bf16 contiguous;
 *  ql_nope [T, N, Lkv] bf16 contiguous output.  fp32 accumulation, one
 *  round-to-nearest-even to bf16.  P a multiple of 32 in [32, 256]; Lkv a multiple of 128.
 */
int mla_absorb_q(const void* q_nope, const void* W_UK, void* ql_nope, int32_t T, int32_t N,
                 int32_t P, int32_t Lkv, void* stream);

/*
 * mla_up_v -- o[t,h,v] = sum_l o_latent[t,h,l] * W_UV[l,h,v].
 * mla/common.py docstring, "Data-Movement Friendly Approach" (einsum
 * "snl,lnv->snv"); mla_attention, _v_up_proj (bmm (N,B,L)x(N,L,V)).
 *  o_latent [T, N, Lkv] bf16 contiguous; W_UV [Lkv, N, V] bf16 contiguous;
 *  o [T, N, V] bf16 contiguous output.  V a multiple of 32 in [32, 256];
 *  Lkv a multiple of 32.
 */
int mla_up_v(const void* o_latent, const void* W_UV, void* o, int32_t T, int32_t N, int32_t Lkv,
             int32_t V, void* stream);

/*
 * merge_attn_states -- combine two attention states over disjoint key sets.
 * mla/common.py docstring, "Chunked Prefill" (merge of prefix and suffix
 * outputs with their LSE); argument order as the vLLM calls on the pages
 * (output, output_lse, prefix_output, prefix_lse, suffix_output, suffix_lse).
 *   m = max(lse_p, lse_s); w_x = exp(lse_x - m)
 *   out = (w_p*prefix + w_s*suffix) / (w_p + w_s);  out_lse = m + ln(w_p + w_s)
 * Both -inf: out = 0, out_lse = -inf.
 *  out, prefix_o, suffix_o  [T, N, D] contiguous, element type o_dtype
 *                           (MLA_DT_BF16 or MLA_DT_FP32); D a multiple of 8, <= 1024.
 *  prefix_lse, suffix_lse   [T, N] fp32 natural-log; out_lse [T, N] fp32 or NULL.
 */
int merge_attn_states(void* out, float* out_lse, const void* prefix_o, const float* prefix_lse,
                      const void* suffix_o, const float* suffix_lse, int32_t T, int32_t N,
                      int32_t D, int32_t o_dtype, void* stream);

/*
 * mla_concat_quant_q -- the decode query of an fp8 cache, concatenated and quantised
 * with a static per-tensor scale (vLLM layers/attention/mla_attention, MLAAttention
 * forward, decode branch: with an fp8 KV cache the absorbed query ql_nope and q_pe are
 * concatenated and quantised to float8 with the layer's q_scale before the backend call).
 *
 *   q8[t, h, 0:512]   = e4m3fn(ql_nope[t, h, :] / q_scale)
 *   q8[t, h, 512:576] = e4m3fn(q_pe[t, h, :] / q_scale)
 * Each value: the bf16 input times the fp32 reciprocal of q_scale (rounded once),
 * clamped to [-448, 448], rounded to the nearest OCP e4m3fn value, ties to even.
 *
 *   ql_nope [T, N, 512] bf16, q_pe [T, N, 64] bf16 (strides in elements, multiples of 8),
 *   q8 [T, N, 576] e4m3fn bytes (strides in bytes, multiples of 16); all 16-byte aligned.
 *   q_scale: finite and > 0.
 * Errors: INVALID_ARG for null pointers, bad sizes, strides, alignment or q_scale.
 */
int mla_concat_quant_q(const void* ql_nope, int64_t ql_s_tok, int64_t ql_s_head, const void* q_pe,
                       int64_t qpe_s_tok, int64_t qpe_s_head, float q_scale, void* q8, int64_t q8_s_tok,
                       int64_t q8_s_head, int32_t T, int32_t N, void* stream);

/*
 * mla_concat_and_cache -- writes new latent rows into the paged cache (vLLM mla/common.py,
 * MLACommonImpl forward: "write the latent and rope to kv cache" with concat_and_cache_mla
 * at slot_mapping; for an fp8 cache, quantised with the layer's k_scale).
 *
 * Token i with s = slot_mapping[i] writes cache row (s / page_size, s % page_size):
 *   bf16 cache: [kv_c[i, 0:512] | k_pe[i, 0:64]] copied;
 *   fp8 cache:  each value x -> e4m3fn(clamp(x * (1 / k_scale), -448, 448)), the reciprocal
 *               rounded once to fp32, round to nearest even (the stored value times k_scale
 *               is the cache value the decode reads with kv_scale = k_scale).
 * Slots outside [0, num_pages * page_size) are skipped; negative slots mark padding
 * tokens.  Two tokens with the same slot: one of them wins (unspecified which).
 *
 *  kv_c [T, 512] bf16 (token stride kv_c_s_tok), k_pe [T, 64] bf16 (k_pe_s_tok),
 *  slot_mapping [T] int64 (device), cache [num_pages, page_size, 576] (strides in
 *  elements of the cache dtype; page stride >= page_size * token stride), cache_dtype
 *  MLA_DT_BF16 or MLA_DT_FP8_E4M3FN, k_scale finite and > 0 for fp8 (unused for bf16).
 *  Rows and strides 16-byte aligned.
 * Errors: INVALID_ARG (nulls, sizes, strides, alignment, k_scale), UNSUPPORTED (dtype), HIP.
 */
int mla_concat_and_cache(const void* kv_c, int64_t kv_c_s_tok, const void* k_pe, int64_t k_pe_s_tok,
                         const int64_t* slot_mapping, int32_t T, void* cache, int64_t cache_s_page,
                         int64_t cache_s_tok, int32_t page_size, int32_t num_pages, int32_t cache_dtype,
                         float k_scale, void* stream);

/* ---- chunked prefill, compute-friendly form ----
 *
 * vLLM mla/common.py module docstring, "Chunked Prefill": keys and values are
 * up-projected per head from the latent rows (k_nope = kv_c W_UK, v = kv_c W_UV),
 * k_pe is shared by all heads, and each head runs attention with QK width P+R and
 * value width V.  The context is visited in chunks (MLACommonImpl.
 * _compute_prefill_context: gather and dequantise the chunk's cache rows, kv_b_proj,
 * attention without a mask), chunk outputs are combined by merge_attn_states, and
 * the new tokens attend to themselves causally (forward_mha), the last merge taking
 * the context output as prefix and the new tokens' output as suffix.
 * Supported: Lkv = 512, R = 64, P = V = 128 (DeepSeek-V3 head dims).
 */

/*
 * mla_prefill_attention -- per-head softmax attention of requests laid out back to
 * back.  Request b owns queries cu_q[b]..cu_q[b+1]-1 and keys cu_k[b]..cu_k[b+1]-1
 * (cu_q, cu_k: device int32 [B+1], non-decreasing from 0); causal != 0: query i of
 * the request (0-based) sees keys j <= i + Sk_b - Sq_b (the new tokens are the last
 * keys), otherwise all Sk_b keys.
 *  q_nope [T,N,P], q_pe [T,N,R], k_nope [S,N,P], k_pe [S,R] (one rope row per key,
 *  shared by the heads), v [S,N,V]: bf16, strides in elements (token, head), rows
 *  16-byte aligned; key and value token strides below 2^25 elements.  max_q >= max_b Sq_b.
 *  scale (finite, > 0) multiplies the logits.
 *  o [T,N,V] bf16 receives sum softmax * v; lse [T,N] fp32 (t*N + h, natural log,
 *  scale included) or NULL.  A query with no key gets o = 0, lse = -inf.
 * Errors: INVALID_ARG (null pointers, strides, alignment), UNSUPPORTED (P, R, V),
 * HIP.  Enqueued on stream; no allocation, no host synchronisation.
 */
int mla_prefill_attention(const void* q_nope, int64_t q_nope_s_tok, int64_t q_nope_s_head, const void* q_pe,
                          int64_t q_pe_s_tok, int64_t q_pe_s_head, const void* k_nope, int64_t k_nope_s_tok,
                          int64_t k_nope_s_head, const void* k_pe, int64_t k_pe_s_tok, const void* v,
                          int64_t v_s_tok, int64_t v_s_head, const int32_t* cu_q, const int32_t* cu_k, int32_t B,
                          int32_t max_q, int32_t N, int32_t P, int32_t R, int32_t V, int32_t causal, float scale,
                          void* o, int64_t o_s_tok, int64_t o_s_head, float* lse, void* stream);

/*
 * mla_gather_context -- one context chunk of the paged cache into contiguous rows
 * (mla/common.py, _compute_prefill_context: gather_and_maybe_dequant_cache).
 * Output row r, for the request b with cu[b] <= r < cu[b+1], is context position
 * p = starts[b] + r - cu[b] of that request: cache row
 * block_table[b][p / page_size], slot p % page_size.  out_kv_c [total,512] and
 * out_k_pe [total,64] bf16 (row strides in elements); fp8 caches are widened and
 * multiplied by kv_scale in fp32, then rounded to bf16 (nearest even).
 * starts [B], cu [B+1]: device int32.  Cache pointers and strides as mla_decode_run.
 * Block-table entries of the positions read must be valid pages (not checked).
 */
int mla_gather_context(const void* cache_kv_c, const void* cache_k_pe, int64_t cache_s_page, int64_t cache_s_tok,
                       int32_t page_size, int32_t kv_dtype, float kv_scale, const int32_t* block_table,
                       int64_t block_table_s_req, const int32_t* starts, const int32_t* cu, int32_t B,
                       int64_t total, void* out_kv_c, int64_t out_kv_c_s_tok, void* out_k_pe,
                       int64_t out_k_pe_s_tok, void* stream);

/*
 * mla_kv_b_proj -- k_nope[s,h,p] = sum_l kv_c[s,l] W_UK[l,h,p] and
 * v[s,h,c] = sum_l kv_c[s,l] W_UV[l,h,c] (the docstring's kv_b_proj split into its
 * W_UK and W_UV parts): kv_c [S,Lkv] bf16 (row stride kv_c_s_tok), W_UK [Lkv,N,P],
 * W_UV [Lkv,N,V], k_nope [S,N,P], v [S,N,V] contiguous bf16; fp32 accumulation,
 * outputs rounded to nearest even.
 */
int mla_kv_b_proj(const void* kv_c, int64_t kv_c_s_tok, const void* W_UK, const void* W_UV, void* k_nope,
                  void* v, int32_t S, int32_t N, int32_t Lkv, int32_t P, int32_t V, void* stream);

/*
 * mla_chunked_prefill_workspace_size -- bytes of device workspace mla_chunked_prefill
 * needs for these host counts (new tokens and context tokens per request), head
 * shape and context workspace of workspace_tokens latent rows.
 * The chunk schedule (MLACommonMetadataBuilder, chunked context): with k requests
 * that have context, mcc = workspace_tokens / k rounded down to a multiple of
 * page_size (kept when smaller than a page); chunk i of request b covers context
 * positions [i*mcc, min((i+1)*mcc, ctx_lens[b])).  WORKSPACE if mcc would be 0.
 */
int mla_chunked_prefill_workspace_size(const int32_t* new_lens_host, const int32_t* ctx_lens_host, int32_t B,
                                       int32_t N, int32_t P, int32_t V, int32_t page_size,
                                       int64_t workspace_tokens, size_t* workspace_bytes_out);

/*
 * mla_chunked_prefill -- output of a prefill batch: request b has ctx_lens[b] tokens
 * of context in the paged cache and new_lens[b] new tokens (rows laid out back to
 * back in request order, T = sum new_lens); new token i of request b sees every
 * context key and the new keys 0..i.
 *  q_nope [T,N,P], q_pe [T,N,R], kv_c [T,Lkv], k_pe [T,R]: the new tokens' queries
 *  and latent rows, contiguous bf16.  new_lens_host, ctx_lens_host: host int32 [B].
 *  Cache, block_table, kv_dtype and kv_scale as mla_decode_run.  W_UK, W_UV
 *  [Lkv,N,P] / [Lkv,N,V] contiguous bf16.  o [T,N,V] bf16 contiguous; lse [T,N] or
 *  NULL.  workspace: device, 256-byte aligned, of the size above.
 * Launches, in order: kv_b_proj and causal attention of the new tokens (into o and
 * lse, or a workspace LSE, as the running state), then per chunk gather, kv_b_proj
 * and attention, whose epilogue merges its result into the running state by LSE
 * (the merge is associative: the pages' order up to the bf16 rounding of the
 * intermediate states); all on stream.  The chunk schedule goes to the workspace by one host-to-device copy
 * from pageable memory.  Errors as the calls above, WORKSPACE if too small.
 */
int mla_chunked_prefill(const void* q_nope, const void* q_pe, const void* kv_c, const void* k_pe,
                        const int32_t* new_lens_host, const int32_t* ctx_lens_host, int32_t B, const void* cache_kv_c,
                        const void* cache_k_pe, int64_t cache_s_page, int64_t cache_s_tok, int32_t page_size,
                        int32_t kv_dtype, float kv_scale, const int32_t* block_table, int64_t block_table_s_req,
                        const void* W_UK, const void* W_UV, int32_t N, int32_t Lkv, int32_t P, int32_t R,
                        int32_t V, float scale, int64_t workspace_tokens, void* o, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---- fp8 W_UK / W_UV BMMs ----
 *
 * vLLM mla/common.py and mla_attention, process_weights_after_loading with the ROCm
 * fp8 BMM: the weights are laid out per head, W_K = W_UK as [N, Lkv, P] and
 * W_V = W_UV as [N, V, Lkv], quantised to e4m3fn with one scale for the whole tensor;
 * the absorption and the up-projection quantise their activations per token in
 * groups of 128 along the contracted dimension and run an fp8 batched GEMM.
 */

/*
 * mla_quant_weight_fp8 -- one weight tensor to fp8, once, at load time.
 *  W      bf16 [Lkv, N, X], contiguous: W_UK (X = P, which = 0) or W_UV (X = V, which = 1).
 *  W8     e4m3fn bytes, written as W_K [N, Lkv, P] (which = 0) or W_V [N, V, Lkv] (which = 1).
 *  w_scale  device fp32[1] receiving the dequantisation scale.
 * Arithmetic (the page's, on bf16 tensors: fp32 compute, bf16 rounding to nearest even):
 * amax = max |W| (at least 1e-10), s = bf16(448 / amax), y = bf16(W * s) clamped to
 * +-448, W8 = e4m3fn(y) to nearest even; w_scale = fp32(1 / s).  Runs as one workgroup
 * (no atomics, no scratch memory); one-time work, not on the per-step path.
 */
int mla_quant_weight_fp8(const void* W, int32_t Lkv, int32_t N, int32_t X, int32_t which, void* W8,
                         float* w_scale, void* stream);

/*
 * mla_absorb_q_fp8 -- ql_nope[t,h,l] = w_scale * sum_g d[t,h,g] sum_{p in g} q8[t,h,p] W_K[h,l,p]
 * mla_up_v_fp8     -- o[t,h,v]       = w_scale * sum_g d[t,h,g] sum_{l in g} x8[t,h,l] W_V[h,v,l]
 *  Activations (q_nope [T,N,P] / o_latent [T,N,Lkv], contiguous bf16) are quantised in
 *  groups g of 128 contracted elements per (token, head) (the page's "a per token group
 *  prequant", group_size 128; its arithmetic is not printed, reading taken: the weights'
 *  formula in fp32): amax = max |a| (at least 1e-10), s = 448 / amax, codes =
 *  e4m3fn(clamp(a * s, +-448)) to nearest even, d = 1 / s.  Weights and w_scale as
 *  written by mla_quant_weight_fp8.  Outputs contiguous bf16, fp32 accumulation.
 *  P (absorb) and Lkv (up) must be multiples of 128.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.  No allocation, no host synchronisation.
 */
int mla_absorb_q_fp8(const void* q_nope, const void* W_K, const float* w_scale, void* ql_nope, int32_t T,
                     int32_t N, int32_t P, int32_t Lkv, void* stream);
int mla_up_v_fp8(const void* o_latent, const void* W_V, const float* w_scale, void* o, int32_t T, int32_t N,
                 int32_t Lkv, int32_t V, void* stream);

/* Text of the calling thread's last non-OK status ("" if none). */
const char* mla_last_error(void);

/* ---- host-only and test exports (integer work, compared bit-exactly) ---- */

/*
 * mla_plan_compute_host -- the plan rule of mla_decode_plan on the host only
 * (no HIP call).  Writes up to *n_items work items of 5 int32 each
 * (part, request, kv_start, kv_end, partial slot or -1), ordered by part, and
 * up to *n_reduce reduce entries of 3 int32 (request, first partial slot,
 * count).  On return *n_items / *n_reduce hold the true counts; if a buffer
 * is NULL or too small only the counts are returned.  *num_parts and
 * *num_partials receive the part and partial-slot counts.
 */
int mla_plan_compute_host(const int32_t* seq_lens_host, int32_t B, int32_t Sq, int32_t N,
                          int32_t num_cus, int32_t* work_host, int32_t* n_items,
                          int32_t* reduce_host, int32_t* n_reduce, int32_t* num_parts,
                          int32_t* num_partials);

/* Copies a plan's work items and reduce entries (formats as above) to host memory. */
int mla_plan_export(mla_plan plan, int32_t* work_host, int32_t* n_items, int32_t* reduce_host,
                    int32_t* n_reduce);

/*
 * mla_debug_gather_rows -- the physical cache row the decode kernel computes for
 * every key: rows_out[off_b + j] = block_table[b][j/page_size]*page_size + j%page_size
 * for j < seq_lens[b], request-major (off_b = sum of earlier seq_lens).  Uses the
 * plan's seq_lens and page_size.  rows_out: device int64 [sum seq_lens].
 */
int mla_debug_gather_rows(mla_plan plan, const int32_t* block_table, int64_t block_table_s_req,
                          int64_t* rows_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_DECODE_H */
