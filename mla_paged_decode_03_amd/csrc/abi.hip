// C ABI of the library: argument validation, plans, launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include <mutex>

#include "../../include/mla_decode.h"
#include "kernels.h"
#include "plan.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Workspace of mla_decode_run_noalloc: a static device array, one copy per device, held
// until the process ends.  In host code `scratch` is only a stand-in symbol; its device
// address comes from hipGetSymbolAddress, resolved once per device with that device
// current and kept in g_scratch.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

struct mla_plan_s {
  mla::Plan host;
  int32_t Lkv = 0, R = 0, page_size = 0, max_pages = 0, kv_dtype = 0;
  std::vector<int32_t> seq_lens;
  int64_t total_keys = 0;
  size_t ws_bytes = 0;
  hipStream_t stream = nullptr;
  int device = 0;
  int32_t* d_buf = nullptr;  // segs | part_begin | reduce | seq_lens | pad | offsets (int64)
  int32_t* h_buf = nullptr;  // pinned staging of the same words
  size_t words = 0;
  size_t off_part = 0, off_reduce = 0, off_seq = 0, off_offsets = 0;
};

extern "C" {

const char* mla_last_error(void) { return g_err.c_str(); }

static int check_workspace(mla_plan plan, void* workspace, size_t workspace_bytes);

static int validate_dims(int32_t B, int32_t Sq, int32_t N, int32_t Lkv, int32_t R, int32_t page_size,
                         int32_t max_pages, int32_t kv_dtype) {
  if (B < 1) return fail(MLA_ERR_INVALID_ARG, "B must be >= 1");
  if (page_size < 1) return fail(MLA_ERR_INVALID_ARG, "page_size must be >= 1");
  if (max_pages < 1) return fail(MLA_ERR_INVALID_ARG, "max_pages_per_req must be >= 1");
  if (Lkv != mla::kLkv || R != mla::kRope)
    return fail(MLA_ERR_UNSUPPORTED, "only Lkv = 512 and R = 64 (head size 576) are supported");
  if (N < 1 || N > 128) return fail(MLA_ERR_UNSUPPORTED, "N must be in [1, 128]");
  if (Sq < 1 || Sq > 8) return fail(MLA_ERR_UNSUPPORTED, "Sq must be in [1, 8]");
  if (kv_dtype != MLA_DT_BF16 && kv_dtype != MLA_DT_FP8_E4M3FN)
    return fail(MLA_ERR_UNSUPPORTED, "kv_dtype must be MLA_DT_BF16 or MLA_DT_FP8_E4M3FN");
  return MLA_OK;
}

int mla_plan_compute_host(const int32_t* seq_lens_host, int32_t B, int32_t Sq, int32_t N,
                          int32_t num_cus, int32_t* work_host, int32_t* n_items,
                          int32_t* reduce_host, int32_t* n_reduce, int32_t* num_parts,
                          int32_t* num_partials) {
  if (!seq_lens_host || !n_items || !n_reduce) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (B < 1 || Sq < 1 || N < 1 || num_cus < 1) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  mla::Plan p;
  std::string err;
  if (!mla::build_plan(seq_lens_host, B, Sq, N, num_cus, &p, &err)) return fail(MLA_ERR_INVALID_ARG, err);
  const int32_t ni = (int32_t)p.segs.size(), nr = (int32_t)p.reduce.size() / 3;
  if (work_host && *n_items >= ni) {
    for (int32_t pt = 0; pt < p.num_parts; ++pt)
      for (int32_t s = p.part_begin[pt]; s < p.part_begin[pt + 1]; ++s) {
        int32_t* o = work_host + 5 * s;
        o[0] = pt;
        o[1] = p.segs[s].req;
        o[2] = p.segs[s].kv_start;
        o[3] = p.segs[s].kv_end;
        o[4] = p.segs[s].partial;
      }
  }
  if (reduce_host && *n_reduce >= nr) std::memcpy(reduce_host, p.reduce.data(), sizeof(int32_t) * 3 * nr);
  *n_items = ni;
  *n_reduce = nr;
  if (num_parts) *num_parts = p.num_parts;
  if (num_partials) *num_partials = p.num_partials;
  return MLA_OK;
}

int mla_decode_plan(const int32_t* seq_lens_host, int32_t B, int32_t Sq, int32_t N, int32_t Lkv,
                    int32_t R, int32_t page_size, int32_t max_pages_per_req, int32_t kv_dtype,
                    int32_t num_cus, void* stream, mla_plan* plan_out,
                    size_t* workspace_bytes_out) {
  if (!seq_lens_host || !plan_out || !workspace_bytes_out) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  *plan_out = nullptr;
  int rc = validate_dims(B, Sq, N, Lkv, R, page_size, max_pages_per_req, kv_dtype);
  if (rc) return rc;
  for (int32_t b = 0; b < B; ++b) {
    if (seq_lens_host[b] < 0) return fail(MLA_ERR_INVALID_ARG, "negative seq_len");
    if (seq_lens_host[b] > mla::kMaxSeqLen) return fail(MLA_ERR_INVALID_ARG, "seq_len above 2^30");
    if ((int64_t)seq_lens_host[b] > (int64_t)max_pages_per_req * page_size)
      return fail(MLA_ERR_INVALID_ARG, "seq_len exceeds max_pages_per_req * page_size");
  }
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (num_cus <= 0) {
    e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  }
  auto* p = new mla_plan_s();
  std::string err;
  if (!mla::build_plan(seq_lens_host, B, Sq, N, num_cus, &p->host, &err)) {
    delete p;
    return fail(MLA_ERR_INTERNAL, err);
  }
  p->Lkv = Lkv;
  p->R = R;
  p->page_size = page_size;
  p->max_pages = max_pages_per_req;
  p->kv_dtype = kv_dtype;
  p->seq_lens.assign(seq_lens_host, seq_lens_host + B);
  p->stream = (hipStream_t)stream;
  p->device = device;
  p->ws_bytes = (size_t)mla::workspace_bytes(p->host.num_partials, Sq, N);

  const size_t nseg = p->host.segs.size();
  p->off_part = 4 * nseg;
  p->off_reduce = p->off_part + p->host.part_begin.size();
  p->off_seq = p->off_reduce + p->host.reduce.size();
  p->off_offsets = (p->off_seq + B + 1) & ~(size_t)1;
  p->words = p->off_offsets + 2 * (size_t)B;
  std::vector<int32_t> w(p->words, 0);
  for (size_t s = 0; s < nseg; ++s) {
    const auto& sg = p->host.segs[s];
    w[4 * s] = sg.req;
    w[4 * s + 1] = sg.kv_start;
    w[4 * s + 2] = sg.kv_end;
    w[4 * s + 3] = sg.partial;
  }
  std::memcpy(&w[p->off_part], p->host.part_begin.data(), 4 * p->host.part_begin.size());
  if (!p->host.reduce.empty()) std::memcpy(&w[p->off_reduce], p->host.reduce.data(), 4 * p->host.reduce.size());
  std::memcpy(&w[p->off_seq], seq_lens_host, 4 * (size_t)B);
  int64_t acc = 0;
  for (int32_t b = 0; b < B; ++b) {
    std::memcpy(&w[p->off_offsets + 2 * b], &acc, 8);
    acc += seq_lens_host[b];
  }
  p->total_keys = acc;

  e = hipMalloc((void**)&p->d_buf, 4 * p->words);
  if (e == hipSuccess) e = hipHostMalloc((void**)&p->h_buf, 4 * p->words, hipHostMallocDefault);
  if (e == hipSuccess) {
    std::memcpy(p->h_buf, w.data(), 4 * p->words);
    e = hipMemcpyAsync(p->d_buf, p->h_buf, 4 * p->words, hipMemcpyHostToDevice, p->stream);
  }
  if (e != hipSuccess) {
    if (p->d_buf) (void)hipFree(p->d_buf);
    if (p->h_buf) (void)hipHostFree(p->h_buf);
    delete p;
    return hip_fail(e, "plan upload");
  }
  *plan_out = p;
  *workspace_bytes_out = p->ws_bytes;
  return MLA_OK;
}

int mla_plan_destroy(mla_plan plan) {
  if (!plan) return MLA_OK;
  hipError_t e = hipStreamSynchronize(plan->stream);
  hipError_t e2 = hipFree(plan->d_buf);
  hipError_t e3 = hipHostFree(plan->h_buf);
  delete plan;
  if (e != hipSuccess) return hip_fail(e, "mla_plan_destroy: stream sync");
  if (e2 != hipSuccess) return hip_fail(e2, "mla_plan_destroy: hipFree");
  if (e3 != hipSuccess) return hip_fail(e3, "mla_plan_destroy: hipHostFree");
  return MLA_OK;
}

int mla_plan_export(mla_plan plan, int32_t* work_host, int32_t* n_items, int32_t* reduce_host,
                    int32_t* n_reduce) {
  if (!plan || !n_items || !n_reduce) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  const auto& p = plan->host;
  const int32_t ni = (int32_t)p.segs.size(), nr = (int32_t)p.reduce.size() / 3;
  if (work_host && *n_items >= ni) {
    for (int32_t pt = 0; pt < p.num_parts; ++pt)
      for (int32_t s = p.part_begin[pt]; s < p.part_begin[pt + 1]; ++s) {
        int32_t* o = work_host + 5 * s;
        o[0] = pt;
        o[1] = p.segs[s].req;
        o[2] = p.segs[s].kv_start;
        o[3] = p.segs[s].kv_end;
        o[4] = p.segs[s].partial;
      }
  }
  if (reduce_host && *n_reduce >= nr) std::memcpy(reduce_host, p.reduce.data(), sizeof(int32_t) * 3 * nr);
  *n_items = ni;
  *n_reduce = nr;
  return MLA_OK;
}

// Queries of one attend call: bf16 q_nope / q_pe, or (q8 != null) fp8 [ql_nope | q_pe]
// with its static scale.
struct Queries {
  const void* q_nope = nullptr;
  int64_t q_nope_s_tok = 0, q_nope_s_head = 0;
  const void* q_pe = nullptr;
  int64_t q_pe_s_tok = 0, q_pe_s_head = 0;
  const void* q8 = nullptr;
  int64_t q8_s_tok = 0, q8_s_head = 0;
  float q_scale = 1.f;
};

static int attend(mla_plan plan, const Queries& q, const void* cache_kv_c, const void* cache_k_pe,
                  int64_t cache_s_page, int64_t cache_s_tok, int32_t num_pages, const int32_t* block_table,
                  int64_t block_table_s_req, const int32_t* seq_lens, float scale, float kv_scale,
                  void* o_latent, int64_t o_s_tok, int64_t o_s_head, float* lse, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARG, "null plan");
  const bool qf8 = q.q8 != nullptr;
  const bool fp8 = plan->kv_dtype == MLA_DT_FP8_E4M3FN;
  if ((!qf8 && (!q.q_nope || !q.q_pe)) || !cache_kv_c || !cache_k_pe || !block_table || !seq_lens || !o_latent)
    return fail(MLA_ERR_INVALID_ARG, "null tensor pointer");
  if (qf8 && !fp8) return fail(MLA_ERR_UNSUPPORTED, "fp8 queries need a plan for an fp8 cache");
  const auto& hp = plan->host;
  if ((!qf8 && (q.q_nope_s_tok < 1 || q.q_nope_s_head < 1 || q.q_pe_s_tok < 1 || q.q_pe_s_head < 1)) ||
      (qf8 && (q.q8_s_head < mla::kHead || q.q8_s_tok < 1)) || o_s_tok < 1 || o_s_head < 1 ||
      cache_s_page < 1 || cache_s_tok < 1 || block_table_s_req < plan->max_pages)
    return fail(MLA_ERR_INVALID_ARG, "bad stride");
  if (qf8 && (!std::isfinite(q.q_scale) || q.q_scale <= 0.f))
    return fail(MLA_ERR_INVALID_ARG, "q_scale must be finite and > 0");
  if (num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages must be >= 1");
  if (!std::isfinite(scale) || !std::isfinite(kv_scale) || scale <= 0.f || kv_scale <= 0.f)
    return fail(MLA_ERR_INVALID_ARG, "scale and kv_scale must be finite and > 0");
  // 16-byte loads of the queries and of cache pieces (8 bf16 or 16 fp8 values), 8-byte
  // output stores; the kernel forms the byte offset of a key within a 32-key tile in 32 bits.
  const size_t cal = 16;
  if (cache_s_tok > (int64_t(1) << 24)) return fail(MLA_ERR_INVALID_ARG, "cache_s_tok too large");
  if (!qf8 && (!aligned(q.q_nope, 16) || !aligned(q.q_pe, 16) || q.q_nope_s_tok % 8 || q.q_nope_s_head % 8 ||
               q.q_pe_s_tok % 8 || q.q_pe_s_head % 8))
    return fail(MLA_ERR_INVALID_ARG, "queries need 16-byte aligned rows (pointer and strides)");
  if (qf8 && (!aligned(q.q8, 16) || q.q8_s_tok % 16 || q.q8_s_head % 16))
    return fail(MLA_ERR_INVALID_ARG, "fp8 queries need 16-byte aligned rows (pointer and strides)");
  const int64_t cel = fp8 ? 16 : 8;  // elements per 16 bytes
  if (!aligned(cache_kv_c, cal) || !aligned(cache_k_pe, cal) || cache_s_page % cel || cache_s_tok % cel)
    return fail(MLA_ERR_INVALID_ARG, "cache rows must be 16-byte aligned (pointers and strides)");
  if (!aligned(o_latent, 16) || o_s_tok % 8 || o_s_head % 8)
    return fail(MLA_ERR_INVALID_ARG, "o_latent needs 16-byte aligned rows (pointer and strides)");
  {
    const int wrc = check_workspace(plan, workspace, workspace_bytes);
    if (wrc) return wrc;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->device) return fail(MLA_ERR_INVALID_ARG, "plan was made for another device");

  mla::DecodeArgs a{};
  a.q_nope = (const uint16_t*)q.q_nope;
  a.q_nope_s_tok = q.q_nope_s_tok;
  a.q_nope_s_head = q.q_nope_s_head;
  a.q_pe = (const uint16_t*)q.q_pe;
  a.q_pe_s_tok = q.q_pe_s_tok;
  a.q_pe_s_head = q.q_pe_s_head;
  a.q8 = (const uint8_t*)q.q8;
  a.q8_s_tok = q.q8_s_tok;
  a.q8_s_head = q.q8_s_head;
  a.kv_c = cache_kv_c;
  a.k_pe = cache_k_pe;
  a.s_page = cache_s_page;
  a.s_tok = cache_s_tok;
  a.block_table = block_table;
  a.bt_s = block_table_s_req;
  a.seq_lens = seq_lens;
  a.segs = plan->d_buf;
  a.part_begin = plan->d_buf + plan->off_part;
  a.o = (uint16_t*)o_latent;
  a.o_s_tok = o_s_tok;
  a.o_s_head = o_s_head;
  a.lse = lse;
  const size_t R = (size_t)hp.Sq * hp.N;
  a.ws_o = workspace;
  a.ws_lse = workspace ? (float*)((char*)workspace + (size_t)hp.num_partials * mla::partial_o_bytes(hp.Sq, hp.N))
                       : nullptr;
  a.ws_l = workspace ? a.ws_lse + (size_t)hp.num_partials * R : nullptr;
  a.qk_scale_log2 = scale * kv_scale * (qf8 ? q.q_scale : 1.f) * 1.4426950408889634f;
  a.out_scale = kv_scale;
  a.Sq = hp.Sq;
  a.N = hp.N;
  a.page_size = plan->page_size;
  a.num_parts = hp.num_parts;
  a.head_groups = hp.head_groups;
  hipStream_t s = (hipStream_t)stream;
  e = mla::launch_decode(a, fp8, qf8, s);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return MLA_OK;
}

int mla_decode_attend(mla_plan plan, const void* q_nope, int64_t q_nope_s_tok, int64_t q_nope_s_head,
                      const void* q_pe, int64_t q_pe_s_tok, int64_t q_pe_s_head,
                      const void* cache_kv_c, const void* cache_k_pe, int64_t cache_s_page,
                      int64_t cache_s_tok, int32_t num_pages, const int32_t* block_table,
                      int64_t block_table_s_req, const int32_t* seq_lens, float scale,
                      float kv_scale, void* o_latent, int64_t o_s_tok, int64_t o_s_head, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream) {
  Queries q;
  q.q_nope = q_nope;
  q.q_nope_s_tok = q_nope_s_tok;
  q.q_nope_s_head = q_nope_s_head;
  q.q_pe = q_pe;
  q.q_pe_s_tok = q_pe_s_tok;
  q.q_pe_s_head = q_pe_s_head;
  return attend(plan, q, cache_kv_c, cache_k_pe, cache_s_page, cache_s_tok, num_pages, block_table,
                block_table_s_req, seq_lens, scale, kv_scale, o_latent, o_s_tok, o_s_head, lse, workspace,
                workspace_bytes, stream);
}

int mla_decode_attend_q8(mla_plan plan, const void* q8, int64_t q8_s_tok, int64_t q8_s_head, float q_scale,
                         const void* cache_kv_c, const void* cache_k_pe, int64_t cache_s_page,
                         int64_t cache_s_tok, int32_t num_pages, const int32_t* block_table,
                         int64_t block_table_s_req, const int32_t* seq_lens, float scale, float kv_scale,
                         void* o_latent, int64_t o_s_tok, int64_t o_s_head, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!q8) return fail(MLA_ERR_INVALID_ARG, "null tensor pointer");
  Queries q;
  q.q8 = q8;
  q.q8_s_tok = q8_s_tok;
  q.q8_s_head = q8_s_head;
  q.q_scale = q_scale;
  return attend(plan, q, cache_kv_c, cache_k_pe, cache_s_page, cache_s_tok, num_pages, block_table,
                block_table_s_req, seq_lens, scale, kv_scale, o_latent, o_s_tok, o_s_head, lse, workspace,
                workspace_bytes, stream);
}

static int check_workspace(mla_plan plan, void* workspace, size_t workspace_bytes) {
  if (plan->ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan->ws_bytes)
      return fail(MLA_ERR_WORKSPACE, "workspace smaller than the plan requires (" +
                                         std::to_string(plan->ws_bytes) + " bytes)");
    if (!aligned(workspace, 16)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  return MLA_OK;
}

int mla_decode_reduce(mla_plan plan, void* o_latent, int64_t o_s_tok, int64_t o_s_head, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARG, "null plan");
  if (!o_latent) return fail(MLA_ERR_INVALID_ARG, "null o_latent");
  if (o_s_tok < 1 || o_s_head < 1) return fail(MLA_ERR_INVALID_ARG, "bad stride");
  if (!aligned(o_latent, 16) || o_s_tok % 8 || o_s_head % 8)
    return fail(MLA_ERR_INVALID_ARG, "o_latent needs 16-byte aligned rows for the merge");
  const int rc = check_workspace(plan, workspace, workspace_bytes);
  if (rc) return rc;
  const auto& hp = plan->host;
  const size_t R = (size_t)hp.Sq * hp.N;
  mla::MergeArgs m{};
  m.reduce = plan->d_buf + plan->off_reduce;
  m.n_reduce = (int32_t)hp.reduce.size() / 3;
  m.ws_o = workspace;
  m.ws_lse = workspace ? (float*)((char*)workspace + (size_t)hp.num_partials * mla::partial_o_bytes(hp.Sq, hp.N))
                       : nullptr;
  m.ws_l = workspace ? m.ws_lse + (size_t)hp.num_partials * R : nullptr;
  m.o = (uint16_t*)o_latent;
  m.o_s_tok = o_s_tok;
  m.o_s_head = o_s_head;
  m.lse = lse;
  m.Sq = hp.Sq;
  m.N = hp.N;
  hipError_t e = mla::launch_split_merge(m, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return MLA_OK;
}

int mla_decode_run(mla_plan plan, const void* q_nope, int64_t q_nope_s_tok, int64_t q_nope_s_head,
                   const void* q_pe, int64_t q_pe_s_tok, int64_t q_pe_s_head,
                   const void* cache_kv_c, const void* cache_k_pe, int64_t cache_s_page,
                   int64_t cache_s_tok, int32_t num_pages, const int32_t* block_table,
                   int64_t block_table_s_req, const int32_t* seq_lens, float scale,
                   float kv_scale, void* o_latent, int64_t o_s_tok, int64_t o_s_head, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int rc = mla_decode_attend(plan, q_nope, q_nope_s_tok, q_nope_s_head, q_pe, q_pe_s_tok, q_pe_s_head,
                             cache_kv_c, cache_k_pe, cache_s_page, cache_s_tok, num_pages, block_table,
                             block_table_s_req, seq_lens, scale, kv_scale, o_latent, o_s_tok, o_s_head,
                             lse, workspace, workspace_bytes, stream);
  if (rc) return rc;
  if (plan->host.reduce.empty()) return MLA_OK;
  return mla_decode_reduce(plan, o_latent, o_s_tok, o_s_head, lse, workspace, workspace_bytes, stream);
}

// Device address of the static scratch on the current device (resolved on first use).
static int static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device index beyond the static scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MLA_ERR_INTERNAL, "static scratch has no device address");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MLA_OK;
}

int mla_decode_run_noalloc(mla_plan plan, const void* q_nope, int64_t q_nope_s_tok, int64_t q_nope_s_head,
                           const void* q_pe, int64_t q_pe_s_tok, int64_t q_pe_s_head, const void* cache_kv_c,
                           const void* cache_k_pe, int64_t cache_s_page, int64_t cache_s_tok, int32_t num_pages,
                           const int32_t* block_table, int64_t block_table_s_req, const int32_t* seq_lens,
                           float scale, float kv_scale, void* o_latent, int64_t o_s_tok, int64_t o_s_head,
                           float* lse, void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARG, "null plan");
  if (plan->ws_bytes > kStaticScratchBytes)
    return fail(MLA_ERR_WORKSPACE, "the plan needs " + std::to_string(plan->ws_bytes) +
                                       " bytes of workspace; the static scratch holds " +
                                       std::to_string(kStaticScratchBytes) + " (use mla_decode_run)");
  void* ws = nullptr;
  if (plan->ws_bytes > 0) {
    const int rc = static_scratch(&ws);
    if (rc) return rc;
  }
  return mla_decode_run(plan, q_nope, q_nope_s_tok, q_nope_s_head, q_pe, q_pe_s_tok, q_pe_s_head, cache_kv_c,
                        cache_k_pe, cache_s_page, cache_s_tok, num_pages, block_table, block_table_s_req, seq_lens,
                        scale, kv_scale, o_latent, o_s_tok, o_s_head, lse, ws, plan->ws_bytes, stream);
}

int mla_decode_run_q8(mla_plan plan, const void* q8, int64_t q8_s_tok, int64_t q8_s_head, float q_scale,
                      const void* cache_kv_c, const void* cache_k_pe, int64_t cache_s_page, int64_t cache_s_tok,
                      int32_t num_pages, const int32_t* block_table, int64_t block_table_s_req,
                      const int32_t* seq_lens, float scale, float kv_scale, void* o_latent, int64_t o_s_tok,
                      int64_t o_s_head, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = mla_decode_attend_q8(plan, q8, q8_s_tok, q8_s_head, q_scale, cache_kv_c, cache_k_pe, cache_s_page,
                                cache_s_tok, num_pages, block_table, block_table_s_req, seq_lens, scale, kv_scale,
                                o_latent, o_s_tok, o_s_head, lse, workspace, workspace_bytes, stream);
  if (rc) return rc;
  if (plan->host.reduce.empty()) return MLA_OK;
  return mla_decode_reduce(plan, o_latent, o_s_tok, o_s_head, lse, workspace, workspace_bytes, stream);
}

int mla_absorb_q(const void* q_nope, const void* W_UK, void* ql_nope, int32_t T, int32_t N,
                 int32_t P, int32_t Lkv, void* stream) {
  if (!q_nope || !W_UK || !ql_nope) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (T < 0 || N < 1 || P < 8 || Lkv < 8) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  if (P % 8 || Lkv % 8) return fail(MLA_ERR_UNSUPPORTED, "P and Lkv must be multiples of 8");
  if (!aligned(q_nope, 16) || !aligned(W_UK, 16) || !aligned(ql_nope, 16))
    return fail(MLA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  mla::GemmArgs g{};
  g.A = (const uint16_t*)q_nope;  // (h, m=t, k=p) at t*N*P + h*P + p
  g.a_sh = P;
  g.a_sm = (int64_t)N * P;
  g.B = (const uint16_t*)W_UK;  // (h, n=l, k=p) at l*N*P + h*P + p
  g.b_sh = P;
  g.b_sn = (int64_t)N * P;
  g.b_sk = 1;
  g.C = (uint16_t*)ql_nope;  // (h, t, l) at t*N*Lkv + h*Lkv + l
  g.c_sh = Lkv;
  g.c_sm = (int64_t)N * Lkv;
  g.H = N;
  g.M = T;
  g.Nn = Lkv;
  g.K = P;
  hipError_t e = mla::launch_gemm(g, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "absorb launch");
}

int mla_up_v(const void* o_latent, const void* W_UV, void* o, int32_t T, int32_t N, int32_t Lkv,
             int32_t V, void* stream) {
  if (!o_latent || !W_UV || !o) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (T < 0 || N < 1 || V < 8 || Lkv < 8) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  if (V % 8 || Lkv % 8) return fail(MLA_ERR_UNSUPPORTED, "V and Lkv must be multiples of 8");
  if (!aligned(o_latent, 16) || !aligned(W_UV, 16) || !aligned(o, 16))
    return fail(MLA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  mla::GemmArgs g{};
  g.A = (const uint16_t*)o_latent;  // (h, t, k=l) at t*N*Lkv + h*Lkv + l
  g.a_sh = Lkv;
  g.a_sm = (int64_t)N * Lkv;
  g.B = (const uint16_t*)W_UV;  // (h, n=v, k=l) at l*N*V + h*V + v
  g.b_sh = V;
  g.b_sn = 1;
  g.b_sk = (int64_t)N * V;
  g.C = (uint16_t*)o;  // (h, t, v) at t*N*V + h*V + v
  g.c_sh = V;
  g.c_sm = (int64_t)N * V;
  g.H = N;
  g.M = T;
  g.Nn = V;
  g.K = Lkv;
  hipError_t e = mla::launch_gemm(g, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "up-projection launch");
}

int merge_attn_states(void* out, float* out_lse, const void* prefix_o, const float* prefix_lse,
                      const void* suffix_o, const float* suffix_lse, int32_t T, int32_t N,
                      int32_t D, int32_t o_dtype, void* stream) {
  if (!out || !prefix_o || !prefix_lse || !suffix_o || !suffix_lse)
    return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (T < 0 || N < 1 || D < 8) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  if (D % 8) return fail(MLA_ERR_UNSUPPORTED, "D must be a multiple of 8");
  if (o_dtype != MLA_DT_BF16 && o_dtype != MLA_DT_FP32)
    return fail(MLA_ERR_UNSUPPORTED, "o_dtype must be MLA_DT_BF16 or MLA_DT_FP32");
  if (!aligned(out, 16) || !aligned(prefix_o, 16) || !aligned(suffix_o, 16))
    return fail(MLA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  hipError_t e = mla::launch_merge_two(out, out_lse, prefix_o, prefix_lse, suffix_o, suffix_lse,
                                       (int64_t)T * N, D, o_dtype == MLA_DT_FP32, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "merge launch");
}

int mla_concat_quant_q(const void* ql_nope, int64_t ql_s_tok, int64_t ql_s_head, const void* q_pe,
                       int64_t qpe_s_tok, int64_t qpe_s_head, float q_scale, void* q8, int64_t q8_s_tok,
                       int64_t q8_s_head, int32_t T, int32_t N, void* stream) {
  if (!ql_nope || !q_pe || !q8) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (T < 0 || N < 1) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  if (!(q_scale > 0.f) || !std::isfinite(q_scale)) return fail(MLA_ERR_INVALID_ARG, "q_scale must be finite and > 0");
  if (ql_s_head < mla::kLkv || ql_s_tok < (int64_t)N * ql_s_head || qpe_s_head < mla::kRope ||
      qpe_s_tok < (int64_t)N * qpe_s_head || q8_s_head < mla::kHead || q8_s_tok < (int64_t)N * q8_s_head)
    return fail(MLA_ERR_INVALID_ARG, "bad stride");
  if (!aligned(ql_nope, 16) || !aligned(q_pe, 16) || !aligned(q8, 16) || ql_s_tok % 8 || ql_s_head % 8 ||
      qpe_s_tok % 8 || qpe_s_head % 8 || q8_s_tok % 16 || q8_s_head % 16)
    return fail(MLA_ERR_INVALID_ARG, "rows must be 16-byte aligned (pointers and strides)");
  mla::QuantArgs a{};
  a.ql = (const uint16_t*)ql_nope;
  a.ql_s_tok = ql_s_tok;
  a.ql_s_head = ql_s_head;
  a.qpe = (const uint16_t*)q_pe;
  a.qpe_s_tok = qpe_s_tok;
  a.qpe_s_head = qpe_s_head;
  a.q8 = (uint8_t*)q8;
  a.q8_s_tok = q8_s_tok;
  a.q8_s_head = q8_s_head;
  a.inv_scale = 1.0f / q_scale;
  a.T = T;
  a.N = N;
  hipError_t e = mla::launch_concat_quant_q(a, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "quant launch");
}

int mla_concat_and_cache(const void* kv_c, int64_t kv_c_s_tok, const void* k_pe, int64_t k_pe_s_tok,
                         const int64_t* slot_mapping, int32_t T, void* cache, int64_t cache_s_page,
                         int64_t cache_s_tok, int32_t page_size, int32_t num_pages, int32_t cache_dtype,
                         float k_scale, void* stream) {
  if (!kv_c || !k_pe || !slot_mapping || !cache) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (T < 0 || page_size < 1 || num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  if (cache_dtype != MLA_DT_BF16 && cache_dtype != MLA_DT_FP8_E4M3FN)
    return fail(MLA_ERR_UNSUPPORTED, "cache_dtype must be MLA_DT_BF16 or MLA_DT_FP8_E4M3FN");
  const bool fp8 = cache_dtype == MLA_DT_FP8_E4M3FN;
  if (fp8 && (!std::isfinite(k_scale) || k_scale <= 0.f))
    return fail(MLA_ERR_INVALID_ARG, "k_scale must be finite and > 0");
  if (kv_c_s_tok < mla::kLkv || k_pe_s_tok < mla::kRope || cache_s_tok < mla::kHead ||
      cache_s_page < (int64_t)page_size * cache_s_tok)
    return fail(MLA_ERR_INVALID_ARG, "bad stride");
  const int64_t cel = fp8 ? 16 : 8;  // elements per 16 bytes
  if (!aligned(kv_c, 16) || !aligned(k_pe, 16) || !aligned(cache, 16) || kv_c_s_tok % 8 || k_pe_s_tok % 8 ||
      cache_s_tok % cel || cache_s_page % cel)
    return fail(MLA_ERR_INVALID_ARG, "rows must be 16-byte aligned (pointers and strides)");
  mla::CacheWriteArgs a{};
  a.kv_c = (const uint16_t*)kv_c;
  a.kv_c_s_tok = kv_c_s_tok;
  a.k_pe = (const uint16_t*)k_pe;
  a.k_pe_s_tok = k_pe_s_tok;
  a.slot_mapping = slot_mapping;
  a.cache = cache;
  a.s_page = cache_s_page;
  a.s_tok = cache_s_tok;
  a.inv_scale = fp8 ? 1.0f / k_scale : 1.f;
  a.T = T;
  a.page_size = page_size;
  a.num_pages = num_pages;
  hipError_t e = mla::launch_cache_write(a, fp8, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "cache-write launch");
}

int mla_debug_gather_rows(mla_plan plan, const int32_t* block_table, int64_t block_table_s_req,
                          int64_t* rows_out, void* stream) {
  if (!plan || !block_table || !rows_out) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (block_table_s_req < plan->max_pages) return fail(MLA_ERR_INVALID_ARG, "bad stride");
  hipError_t e = mla::launch_gather_rows(block_table, block_table_s_req, plan->d_buf + plan->off_seq,
                                         (const int64_t*)(plan->d_buf + plan->off_offsets), plan->host.B,
                                         plan->page_size, rows_out, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "gather-rows launch");
}

// ---------------------------------------------------------------------------------
// Chunked prefill (compute-friendly form)
// ---------------------------------------------------------------------------------

// Prefill attention; with prev_o / prev_lse the output is the LSE merge of that running
// state (same layouts as o / lse, may alias them) with this launch's attention.
static int prefill_attention_impl(const void* q_nope, int64_t q_nope_s_tok, int64_t q_nope_s_head,
                                  const void* q_pe, int64_t q_pe_s_tok, int64_t q_pe_s_head, const void* k_nope,
                                  int64_t k_nope_s_tok, int64_t k_nope_s_head, const void* k_pe,
                                  int64_t k_pe_s_tok, const void* v, int64_t v_s_tok, int64_t v_s_head,
                                  const int32_t* cu_q, const int32_t* cu_k, int32_t B, int32_t max_q, int32_t N,
                                  int32_t P, int32_t R, int32_t V, int32_t causal, float scale, void* o,
                                  int64_t o_s_tok, int64_t o_s_head, float* lse, const void* prev_o,
                                  const float* prev_lse, void* stream) {
  if (!q_nope || !q_pe || !k_nope || !k_pe || !v || !cu_q || !cu_k || !o)
    return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (B < 0 || max_q < 0 || N < 1) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  if ((int64_t)((max_q + 127) / 128) * N * B > (int64_t)INT32_MAX - 8)
    return fail(MLA_ERR_UNSUPPORTED, "too many (request, head, query block) items");
  if (P != 128 || R != mla::kRope || V != 128)
    return fail(MLA_ERR_UNSUPPORTED, "only P = 128, R = 64 and V = 128 are supported");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(MLA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (q_nope_s_head < P || q_pe_s_head < R || k_nope_s_head < P || v_s_head < V || o_s_head < V ||
      q_nope_s_tok < (int64_t)N * q_nope_s_head || q_pe_s_tok < (int64_t)N * q_pe_s_head ||
      k_nope_s_tok < (int64_t)N * k_nope_s_head || k_pe_s_tok < R || v_s_tok < (int64_t)N * v_s_head ||
      o_s_tok < (int64_t)N * o_s_head)
    return fail(MLA_ERR_INVALID_ARG, "bad stride");
  // the kernel addresses a tile's rows by 32-bit byte offsets from a per-tile base
  if (k_nope_s_tok >= (1 << 25) || k_pe_s_tok >= (1 << 25) || v_s_tok >= (1 << 25))
    return fail(MLA_ERR_UNSUPPORTED, "key / value token strides must be below 2^25 elements");
  const int64_t st[] = {q_nope_s_tok, q_nope_s_head, q_pe_s_tok, q_pe_s_head, k_nope_s_tok, k_nope_s_head,
                        k_pe_s_tok, v_s_tok, v_s_head, o_s_tok, o_s_head};
  for (int64_t x : st)
    if (x % 8) return fail(MLA_ERR_INVALID_ARG, "rows must be 16-byte aligned (strides)");
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(k_nope, 16) || !aligned(k_pe, 16) ||
      !aligned(v, 16) || !aligned(o, 16))
    return fail(MLA_ERR_INVALID_ARG, "rows must be 16-byte aligned (pointers)");
  mla::PrefillAttnArgs a{};
  a.q_nope = (const uint16_t*)q_nope;
  a.qn_s_tok = q_nope_s_tok;
  a.qn_s_head = q_nope_s_head;
  a.q_pe = (const uint16_t*)q_pe;
  a.qp_s_tok = q_pe_s_tok;
  a.qp_s_head = q_pe_s_head;
  a.k_nope = (const uint16_t*)k_nope;
  a.kn_s_tok = k_nope_s_tok;
  a.kn_s_head = k_nope_s_head;
  a.k_pe = (const uint16_t*)k_pe;
  a.kp_s_tok = k_pe_s_tok;
  a.v = (const uint16_t*)v;
  a.v_s_tok = v_s_tok;
  a.v_s_head = v_s_head;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.o = (uint16_t*)o;
  a.o_s_tok = o_s_tok;
  a.o_s_head = o_s_head;
  a.lse = lse;
  a.prev_o = (const uint16_t*)prev_o;
  a.prev_lse = prev_lse;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.N = N;
  a.causal = causal ? 1 : 0;
  hipError_t e = mla::launch_prefill_attn(a, B, max_q, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "prefill attention launch");
}

int mla_prefill_attention(const void* q_nope, int64_t q_nope_s_tok, int64_t q_nope_s_head, const void* q_pe,
                          int64_t q_pe_s_tok, int64_t q_pe_s_head, const void* k_nope, int64_t k_nope_s_tok,
                          int64_t k_nope_s_head, const void* k_pe, int64_t k_pe_s_tok, const void* v,
                          int64_t v_s_tok, int64_t v_s_head, const int32_t* cu_q, const int32_t* cu_k, int32_t B,
                          int32_t max_q, int32_t N, int32_t P, int32_t R, int32_t V, int32_t causal, float scale,
                          void* o, int64_t o_s_tok, int64_t o_s_head, float* lse, void* stream) {
  return prefill_attention_impl(q_nope, q_nope_s_tok, q_nope_s_head, q_pe, q_pe_s_tok, q_pe_s_head, k_nope,
                                k_nope_s_tok, k_nope_s_head, k_pe, k_pe_s_tok, v, v_s_tok, v_s_head, cu_q, cu_k, B,
                                max_q, N, P, R, V, causal, scale, o, o_s_tok, o_s_head, lse, nullptr, nullptr,
                                stream);
}

int mla_gather_context(const void* cache_kv_c, const void* cache_k_pe, int64_t cache_s_page, int64_t cache_s_tok,
                       int32_t page_size, int32_t kv_dtype, float kv_scale, const int32_t* block_table,
                       int64_t block_table_s_req, const int32_t* starts, const int32_t* cu, int32_t B,
                       int64_t total, void* out_kv_c, int64_t out_kv_c_s_tok, void* out_k_pe,
                       int64_t out_k_pe_s_tok, void* stream) {
  if (!cache_kv_c || !cache_k_pe || !block_table || !starts || !cu || !out_kv_c || !out_k_pe)
    return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (B < 1 || total < 0 || page_size < 1) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  if (kv_dtype != MLA_DT_BF16 && kv_dtype != MLA_DT_FP8_E4M3FN)
    return fail(MLA_ERR_UNSUPPORTED, "kv_dtype must be MLA_DT_BF16 or MLA_DT_FP8_E4M3FN");
  const bool fp8 = kv_dtype == MLA_DT_FP8_E4M3FN;
  if (fp8 && (!std::isfinite(kv_scale) || kv_scale <= 0.f))
    return fail(MLA_ERR_INVALID_ARG, "kv_scale must be finite and > 0");
  if (cache_s_tok < mla::kHead || cache_s_page < (int64_t)page_size * cache_s_tok || out_kv_c_s_tok < mla::kLkv ||
      out_k_pe_s_tok < mla::kRope)
    return fail(MLA_ERR_INVALID_ARG, "bad stride");
  const int64_t cel = fp8 ? 8 : 8;  // bf16: 16-byte chunks; fp8: 8-byte chunks of 8 values
  if (!aligned(cache_kv_c, fp8 ? 8 : 16) || !aligned(cache_k_pe, fp8 ? 8 : 16) || !aligned(out_kv_c, 16) ||
      !aligned(out_k_pe, 16) || cache_s_tok % cel || cache_s_page % cel || out_kv_c_s_tok % 8 ||
      out_k_pe_s_tok % 8)
    return fail(MLA_ERR_INVALID_ARG, "rows must be aligned (pointers and strides)");
  mla::GatherArgs a{};
  a.kv_c = cache_kv_c;
  a.k_pe = cache_k_pe;
  a.s_page = cache_s_page;
  a.s_tok = cache_s_tok;
  a.block_table = block_table;
  a.bt_s = block_table_s_req;
  a.starts = starts;
  a.cu = cu;
  a.out_kv_c = (uint16_t*)out_kv_c;
  a.okv_s = out_kv_c_s_tok;
  a.out_k_pe = (uint16_t*)out_k_pe;
  a.ope_s = out_k_pe_s_tok;
  a.kv_scale = fp8 ? kv_scale : 1.f;
  a.total = total;
  a.B = B;
  a.page_size = page_size;
  hipError_t e = mla::launch_gather_ctx(a, fp8, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "context gather launch");
}

int mla_kv_b_proj(const void* kv_c, int64_t kv_c_s_tok, const void* W_UK, const void* W_UV, void* k_nope,
                  void* v, int32_t S, int32_t N, int32_t Lkv, int32_t P, int32_t V, void* stream) {
  if (!kv_c || !W_UK || !W_UV || !k_nope || !v) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (S < 0 || N < 1 || P < 8 || V < 8 || Lkv < 8) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  if (P % 8 || V % 8 || Lkv % 8) return fail(MLA_ERR_UNSUPPORTED, "P, V and Lkv must be multiples of 8");
  if (kv_c_s_tok < Lkv || kv_c_s_tok % 8) return fail(MLA_ERR_INVALID_ARG, "bad stride");
  if (!aligned(kv_c, 16) || !aligned(W_UK, 16) || !aligned(W_UV, 16) || !aligned(k_nope, 16) || !aligned(v, 16))
    return fail(MLA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (S == 0) return MLA_OK;
  hipError_t e;
  if (Lkv % 32 == 0) {
    // one launch over both weights: [S x Lkv] by [Lkv x N*P] and [Lkv x N*V]
    mla::KvbArgs g{};
    g.A = (const uint16_t*)kv_c;
    g.a_s = kv_c_s_tok;
    g.B0 = (const uint16_t*)W_UK;
    g.B1 = (const uint16_t*)W_UV;
    g.C0 = (uint16_t*)k_nope;
    g.C1 = (uint16_t*)v;
    g.N0 = N * P;
    g.N1 = N * V;
    g.M = S;
    g.K = Lkv;
    e = mla::launch_kvb_gemm(g, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kv_b_proj launch");
    return MLA_OK;
  }
  // other latent widths: the per-head GEMM, each head's weight slice against all rows
  for (int which = 0; which < 2; ++which) {
    const int32_t W = which ? V : P;
    mla::GemmArgs g{};
    g.A = (const uint16_t*)kv_c;  // (h, m=s, k=l) at s*kv_c_s_tok + l: shared by the heads
    g.a_sh = 0;
    g.a_sm = kv_c_s_tok;
    g.B = (const uint16_t*)(which ? W_UV : W_UK);  // (h, n, k=l) at l*N*W + h*W + n
    g.b_sh = W;
    g.b_sn = 1;
    g.b_sk = (int64_t)N * W;
    g.C = (uint16_t*)(which ? v : k_nope);  // (h, s, n) at s*N*W + h*W + n
    g.c_sh = W;
    g.c_sm = (int64_t)N * W;
    g.H = N;
    g.M = S;
    g.Nn = W;
    g.K = Lkv;
    e = mla::launch_gemm(g, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kv_b_proj launch");
  }
  return MLA_OK;
}

namespace {

// Chunk schedule of the context (mla/common.py, MLACommonMetadataBuilder, chunked
// context): the workspace is split evenly over the requests that have context, rounded
// down to a multiple of the page size; chunk i of request b covers positions
// [i*mcc, min((i+1)*mcc, C_b)).
struct ChunkSched {
  int64_t mcc = 0;
  int n = 0;
  std::vector<int32_t> starts, cu;  // [n][B], [n][B+1]
  int64_t max_total = 0;
};

int chunk_schedule(const int32_t* ctx, int32_t B, int32_t page_size, int64_t workspace_tokens, ChunkSched& cs) {
  int64_t with_ctx = 0, cmax = 0;
  for (int b = 0; b < B; ++b) {
    if (ctx[b] < 0) return fail(MLA_ERR_INVALID_ARG, "negative context length");
    with_ctx += ctx[b] > 0;
    cmax = std::max<int64_t>(cmax, ctx[b]);
  }
  cs = ChunkSched{};
  if (with_ctx == 0) return MLA_OK;
  int64_t mcc = workspace_tokens / with_ctx;
  if (mcc >= page_size) mcc = mcc / page_size * page_size;
  if (mcc <= 0) return fail(MLA_ERR_WORKSPACE, "workspace_tokens smaller than the number of requests with context");
  cs.mcc = mcc;
  cs.n = (int)((cmax + mcc - 1) / mcc);
  cs.starts.assign((size_t)cs.n * B, 0);
  cs.cu.assign((size_t)cs.n * (B + 1), 0);
  for (int i = 0; i < cs.n; ++i) {
    int64_t acc = 0;
    for (int b = 0; b < B; ++b) {
      const int64_t st = (int64_t)i * mcc, en = std::min<int64_t>(ctx[b], st + mcc);
      cs.starts[(size_t)i * B + b] = (int32_t)st;
      cs.cu[(size_t)i * (B + 1) + b] = (int32_t)acc;
      acc += std::max<int64_t>(0, en - st);
    }
    cs.cu[(size_t)i * (B + 1) + B] = (int32_t)acc;
    cs.max_total = std::max(cs.max_total, acc);
  }
  return MLA_OK;
}

struct PrefillLayout {
  size_t meta, lat_kv, lat_pe, kn, vv, l_run, total;
};

PrefillLayout prefill_layout(int64_t T, int32_t B, int32_t N, int32_t P, int32_t V, const ChunkSched& cs) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  PrefillLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up(bytes);
    return o;
  };
  const int64_t S = std::max<int64_t>(T, cs.max_total);
  const bool ctx = cs.n > 0;
  L.meta = take(sizeof(int32_t) * ((size_t)(B + 1) + (size_t)cs.n * (2 * B + 1)));
  L.lat_kv = take(ctx ? (size_t)cs.max_total * mla::kLkv * 2 : 0);
  L.lat_pe = take(ctx ? (size_t)cs.max_total * mla::kRope * 2 : 0);
  L.kn = take((size_t)S * N * P * 2);
  L.vv = take((size_t)S * N * V * 2);
  L.l_run = take(ctx ? (size_t)T * N * 4 : 0);  // running LSE when the caller passes none
  L.total = off;
  return L;
}

}  // namespace

int mla_chunked_prefill_workspace_size(const int32_t* new_lens_host, const int32_t* ctx_lens_host, int32_t B,
                                       int32_t N, int32_t P, int32_t V, int32_t page_size,
                                       int64_t workspace_tokens, size_t* workspace_bytes_out) {
  if (!new_lens_host || !ctx_lens_host || !workspace_bytes_out) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (B < 1 || N < 1 || page_size < 1 || workspace_tokens < 1) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  int64_t T = 0;
  for (int b = 0; b < B; ++b) {
    if (new_lens_host[b] < 0) return fail(MLA_ERR_INVALID_ARG, "negative new-token count");
    T += new_lens_host[b];
  }
  ChunkSched cs;
  const int rc = chunk_schedule(ctx_lens_host, B, page_size, workspace_tokens, cs);
  if (rc != MLA_OK) return rc;
  *workspace_bytes_out = prefill_layout(T, B, N, P, V, cs).total;
  return MLA_OK;
}

int mla_chunked_prefill(const void* q_nope, const void* q_pe, const void* kv_c, const void* k_pe,
                        const int32_t* new_lens_host, const int32_t* ctx_lens_host, int32_t B, const void* cache_kv_c,
                        const void* cache_k_pe, int64_t cache_s_page, int64_t cache_s_tok, int32_t page_size,
                        int32_t kv_dtype, float kv_scale, const int32_t* block_table, int64_t block_table_s_req,
                        const void* W_UK, const void* W_UV, int32_t N, int32_t Lkv, int32_t P, int32_t R,
                        int32_t V, float scale, int64_t workspace_tokens, void* o, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!q_nope || !q_pe || !kv_c || !k_pe || !new_lens_host || !ctx_lens_host || !W_UK || !W_UV || !o)
    return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (B < 1 || N < 1 || page_size < 1 || workspace_tokens < 1) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  if (Lkv != mla::kLkv || R != mla::kRope || P != 128 || V != 128)
    return fail(MLA_ERR_UNSUPPORTED, "only Lkv = 512, R = 64, P = 128 and V = 128 are supported");
  hipStream_t st = (hipStream_t)stream;
  int64_t T = 0;
  int32_t max_q = 0;
  std::vector<int32_t> meta((size_t)B + 1, 0);
  for (int b = 0; b < B; ++b) {
    if (new_lens_host[b] < 0) return fail(MLA_ERR_INVALID_ARG, "negative new-token count");
    T += new_lens_host[b];
    max_q = std::max(max_q, new_lens_host[b]);
    if (T > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "too many tokens");
    meta[b + 1] = (int32_t)T;
  }
  ChunkSched cs;
  int rc = chunk_schedule(ctx_lens_host, B, page_size, workspace_tokens, cs);
  if (rc != MLA_OK) return rc;
  if (cs.n > 0 && (!cache_kv_c || !cache_k_pe || !block_table)) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  const PrefillLayout L = prefill_layout(T, B, N, P, V, cs);
  if (!workspace || workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace smaller than required (" + std::to_string(L.total) + " bytes)");
  if (!aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (T == 0) return MLA_OK;
  for (int i = 0; i < cs.n; ++i) {
    meta.insert(meta.end(), cs.starts.begin() + (size_t)i * B, cs.starts.begin() + (size_t)(i + 1) * B);
    meta.insert(meta.end(), cs.cu.begin() + (size_t)i * (B + 1), cs.cu.begin() + (size_t)(i + 1) * (B + 1));
  }
  char* ws = (char*)workspace;
  int32_t* d_meta = (int32_t*)(ws + L.meta);
  // pageable source: the copy has read it when the call returns
  hipError_t e = hipMemcpyAsync(d_meta, meta.data(), meta.size() * sizeof(int32_t), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "prefill metadata upload");
  const int32_t* cu_new = d_meta;
  void* kn = ws + L.kn;
  void* vv = ws + L.vv;
  const bool has_ctx = cs.n > 0;

  // new tokens: up-projection of their own latent rows, causal attention among them.  The
  // caller's o (and lse, or a workspace LSE) then hold the running state, into which each
  // context chunk's attention is merged by LSE in its epilogue; the merge is associative, so
  // this equals merging the chunks first and the new tokens last.
  rc = mla_kv_b_proj(kv_c, Lkv, W_UK, W_UV, kn, vv, (int32_t)T, N, Lkv, P, V, stream);
  if (rc != MLA_OK) return rc;
  float* l_run = lse ? lse : (has_ctx ? (float*)(ws + L.l_run) : nullptr);
  rc = prefill_attention_impl(q_nope, (int64_t)N * P, P, q_pe, (int64_t)N * R, R, kn, (int64_t)N * P, P, k_pe, R,
                              vv, (int64_t)N * V, V, cu_new, cu_new, B, max_q, N, P, R, V, 1, scale, o,
                              (int64_t)N * V, V, l_run, nullptr, nullptr, stream);
  if (rc != MLA_OK || !has_ctx) return rc;

  // context chunks: gather (and dequantise), up-project, attend without a mask, merge
  void* lat_kv = ws + L.lat_kv;
  void* lat_pe = ws + L.lat_pe;
  for (int i = 0; i < cs.n; ++i) {
    const int32_t* d_starts = d_meta + (B + 1) + (size_t)i * (2 * B + 1);
    const int32_t* d_cu = d_starts + B;
    const int64_t tot = cs.cu[(size_t)i * (B + 1) + B];
    rc = mla_gather_context(cache_kv_c, cache_k_pe, cache_s_page, cache_s_tok, page_size, kv_dtype, kv_scale,
                            block_table, block_table_s_req, d_starts, d_cu, B, tot, lat_kv, mla::kLkv, lat_pe,
                            mla::kRope, stream);
    if (rc != MLA_OK) return rc;
    rc = mla_kv_b_proj(lat_kv, mla::kLkv, W_UK, W_UV, kn, vv, (int32_t)tot, N, Lkv, P, V, stream);
    if (rc != MLA_OK) return rc;
    rc = prefill_attention_impl(q_nope, (int64_t)N * P, P, q_pe, (int64_t)N * R, R, kn, (int64_t)N * P, P, lat_pe,
                                mla::kRope, vv, (int64_t)N * V, V, cu_new, d_cu, B, max_q, N, P, R, V, 0, scale, o,
                                (int64_t)N * V, V, l_run, o, l_run, stream);
    if (rc != MLA_OK) return rc;
  }
  return MLA_OK;
}

// ---------------------------------------------------------------------------------
// fp8 W_UK / W_UV BMMs
// ---------------------------------------------------------------------------------

int mla_quant_weight_fp8(const void* W, int32_t Lkv, int32_t N, int32_t X, int32_t which, void* W8,
                         float* w_scale, void* stream) {
  if (!W || !W8 || !w_scale) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (Lkv < 1 || N < 1 || X < 8 || X % 8) return fail(MLA_ERR_INVALID_ARG, "bad sizes (X a multiple of 8)");
  if (which != 0 && which != 1) return fail(MLA_ERR_INVALID_ARG, "which must be 0 (W_UK) or 1 (W_UV)");
  if (!aligned(W, 16) || !aligned(W8, 8)) return fail(MLA_ERR_INVALID_ARG, "W must be 16-byte and W8 8-byte aligned");
  hipError_t e = mla::launch_quant_weight((const uint16_t*)W, Lkv, N, X, which, (uint8_t*)W8, w_scale,
                                          (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "weight quantisation launch");
}

int mla_absorb_q_fp8(const void* q_nope, const void* W_K, const float* w_scale, void* ql_nope, int32_t T,
                     int32_t N, int32_t P, int32_t Lkv, void* stream) {
  if (!q_nope || !W_K || !w_scale || !ql_nope) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (T < 0 || N < 1 || P < 128 || Lkv < 8) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  if (P % 128 || Lkv % 8) return fail(MLA_ERR_UNSUPPORTED, "P must be a multiple of 128 and Lkv of 8");
  if (!aligned(q_nope, 16) || !aligned(W_K, 16) || !aligned(ql_nope, 16))
    return fail(MLA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  mla::Bmm8Args g{};
  g.A = (const uint16_t*)q_nope;  // (h, t, p) at t*N*P + h*P + p
  g.a_sh = P;
  g.a_sm = (int64_t)N * P;
  g.B = (const uint8_t*)W_K;  // (h, l, p) at h*Lkv*P + l*P + p
  g.b_sh = (int64_t)Lkv * P;
  g.b_sn = P;
  g.C = (uint16_t*)ql_nope;  // (h, t, l) at t*N*Lkv + h*Lkv + l
  g.c_sh = Lkv;
  g.c_sm = (int64_t)N * Lkv;
  g.w_scale = w_scale;
  g.H = N;
  g.M = T;
  g.Nn = Lkv;
  g.K = P;
  hipError_t e = mla::launch_bmm8(g, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "fp8 absorb launch");
}

int mla_up_v_fp8(const void* o_latent, const void* W_V, const float* w_scale, void* o, int32_t T, int32_t N,
                 int32_t Lkv, int32_t V, void* stream) {
  if (!o_latent || !W_V || !w_scale || !o) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  if (T < 0 || N < 1 || V < 8 || Lkv < 128) return fail(MLA_ERR_INVALID_ARG, "bad sizes");
  if (Lkv % 128 || V % 8) return fail(MLA_ERR_UNSUPPORTED, "Lkv must be a multiple of 128 and V of 8");
  if (!aligned(o_latent, 16) || !aligned(W_V, 16) || !aligned(o, 16))
    return fail(MLA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  mla::Bmm8Args g{};
  g.A = (const uint16_t*)o_latent;  // (h, t, l) at t*N*Lkv + h*Lkv + l
  g.a_sh = Lkv;
  g.a_sm = (int64_t)N * Lkv;
  g.B = (const uint8_t*)W_V;  // (h, v, l) at h*V*Lkv + v*Lkv + l
  g.b_sh = (int64_t)V * Lkv;
  g.b_sn = Lkv;
  g.C = (uint16_t*)o;  // (h, t, v) at t*N*V + h*V + v
  g.c_sh = V;
  g.c_sm = (int64_t)N * V;
  g.w_scale = w_scale;
  g.H = N;
  g.M = T;
  g.Nn = V;
  g.K = Lkv;
  hipError_t e = mla::launch_bmm8(g, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "fp8 up-projection launch");
}

}  // extern "C"
