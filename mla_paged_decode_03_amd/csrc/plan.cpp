// Split-KV work planner.
//
// The ROCm backend on the pages (rocm_aiter_mla, AiterMLAMetadataBuilder)
// fills persistent work and reduce maps once per batch and keeps that work
// off the forward path; its rule is not shown.  This rule is the library's:
// the keys of all requests, counted in 64-key granules, are dealt in request
// order to at most num_cus / head_groups parts of near-equal cost, each
// segment costing kSegCost extra granules for its query load and epilogue.  A
// request cut between parts is computed as partial (o, lse) states that the
// merge kernel combines.
#include "plan.h"

#include <algorithm>

namespace mla {

namespace {

struct Piece {
  int32_t req, g0, g1;
};

// Greedy fill for one cost target; returns the parts as lists of pieces.
void fill(const std::vector<int32_t>& gran, int64_t target, std::vector<std::vector<Piece>>* parts) {
  parts->clear();
  std::vector<Piece> cur;
  int64_t load = 0;
  for (int32_t b = 0; b < (int32_t)gran.size(); ++b) {
    int32_t done = 0;
    for (;;) {
      const int64_t rem = gran[b] - done;
      const int64_t room = target - load - kSegCost;
      if (!cur.empty() && room < std::min<int64_t>(rem, kMinChunk)) {
        parts->push_back(cur);
        cur.clear();
        load = 0;
        continue;
      }
      const int64_t take = std::min(rem, room);
      cur.push_back({b, done, (int32_t)(done + take)});
      load += kSegCost + take;
      done += (int32_t)take;
      if (done == gran[b]) break;
    }
  }
  if (!cur.empty()) parts->push_back(cur);
}

}  // namespace

bool build_plan(const int32_t* seq_lens, int32_t B, int32_t Sq, int32_t N, int32_t num_cus,
                Plan* out, std::string* err) {
  if (!seq_lens || B < 1 || Sq < 1 || N < 1 || num_cus < 1) {
    *err = "build_plan: invalid arguments";
    return false;
  }
  std::vector<int32_t> gran(B);
  int64_t total = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (seq_lens[b] < 0) {
      *err = "build_plan: negative seq_len";
      return false;
    }
    if (seq_lens[b] > kMaxSeqLen) {
      *err = "build_plan: seq_len above the supported maximum (2^30 keys)";
      return false;
    }
    gran[b] = (int32_t)(((int64_t)seq_lens[b] + kGranule - 1) / kGranule);
    total += gran[b] + kSegCost;
  }
  const int32_t hg = head_groups(Sq, N);
  const int64_t budget = std::max<int64_t>(1, num_cus / hg);
  int64_t target = std::max<int64_t>((total + budget - 1) / budget, kSegCost + kMinChunk);
  std::vector<std::vector<Piece>> parts;
  for (;; ++target) {
    fill(gran, target, &parts);
    if ((int64_t)parts.size() <= budget) break;
  }

  std::vector<int32_t> nseg(B, 0);
  for (const auto& p : parts)
    for (const auto& pc : p) ++nseg[pc.req];
  std::vector<int32_t> base(B, -1);
  out->reduce.clear();
  int32_t next = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (nseg[b] > 1) {
      base[b] = next;
      out->reduce.insert(out->reduce.end(), {b, next, nseg[b]});
      next += nseg[b];
    }
  }
  std::vector<int32_t> seen(B, 0);
  out->segs.clear();
  out->part_begin.assign(1, 0);
  for (const auto& p : parts) {
    for (const auto& pc : p) {
      Segment s;
      s.req = pc.req;
      s.kv_start = pc.g0 * kGranule;
      s.kv_end = (int32_t)std::min<int64_t>((int64_t)pc.g1 * kGranule, seq_lens[pc.req]);
      s.partial = nseg[pc.req] > 1 ? base[pc.req] + seen[pc.req]++ : -1;
      out->segs.push_back(s);
    }
    out->part_begin.push_back((int32_t)out->segs.size());
  }
  out->B = B;
  out->Sq = Sq;
  out->N = N;
  out->head_groups = hg;
  out->num_parts = (int32_t)parts.size();
  out->num_partials = next;
  return true;
}

}  // namespace mla
