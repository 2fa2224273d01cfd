// Host-only driver of the split-KV planner for sanitizer runs (test infrastructure).
// Reads cases from stdin, each "B Sq N num_cus" then B seq_lens; for each case prints
// "ok num_parts num_partials n_items n_reduce", then one line per segment
// "part req kv_start kv_end partial" and one per reduce entry "req base count";
// or "err <message>" when the planner rejects the input.
#include <cstdio>
#include <string>
#include <vector>

#include "../../mla_paged_decode_03_amd/csrc/plan.h"

int main() {
  int B, Sq, N, cus;
  while (std::scanf("%d %d %d %d", &B, &Sq, &N, &cus) == 4) {
    std::vector<int32_t> L(B > 0 ? B : 0);
    for (auto& x : L)
      if (std::scanf("%d", &x) != 1) return 2;
    mla::Plan p;
    std::string err;
    if (!mla::build_plan(L.empty() ? nullptr : L.data(), B, Sq, N, cus, &p, &err)) {
      std::printf("err %s\n", err.c_str());
      continue;
    }
    std::printf("ok %d %d %zu %zu\n", p.num_parts, p.num_partials, p.segs.size(), p.reduce.size() / 3);
    for (int pt = 0; pt < p.num_parts; ++pt)
      for (int s = p.part_begin[pt]; s < p.part_begin[pt + 1]; ++s)
        std::printf("%d %d %d %d %d\n", pt, p.segs[s].req, p.segs[s].kv_start, p.segs[s].kv_end, p.segs[s].partial);
    for (size_t i = 0; i < p.reduce.size(); i += 3)
      std::printf("%d %d %d\n", p.reduce[i], p.reduce[i + 1], p.reduce[i + 2]);
  }
  return 0;
}
